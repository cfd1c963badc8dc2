// Prefill GEMM Y = X W^T for packed group-64 W4A16 weights on bf16 MFMA.
//
// The pages' prompt path runs a tiled GEMM on the matrix units with the
// weights dequantized once per tile (aot-llm README, Metal backend notes);
// prompt evaluation is compute-bound where decode is memory-bound (aot-llm
// README, "Batched prompt processing").
//
// gfx950 mapping.  A workgroup of 4 waves owns a BN x BM output tile (BN
// weight rows x BM tokens).  The K loop steps by 64 = one W4A16 group, so
// every weight row has exactly one (scale, zero) per step.  Each step:
//   * the packed nibbles of the BN x 64 weight tile are dequantized once, in
//     f32 (w = s*q - s*z, exact for 4-bit q and fp16 s, z) and rounded to bf16
//     (v_cvt_pk_bf16_f32, round to nearest even) into LDS;
//   * the BM x 64 bf16 activation tile is copied into LDS;
//   * each wave contracts its (BN/WN) x (BM/WM) sub-tile with
//     v_mfma_f32_16x16x32_bf16, A = weight rows, B = token rows, f32
//     accumulators in registers.
// The next step's global loads are issued before the current step's MFMAs
// (register prefetch), so HBM / L2 latency overlaps the matrix work.  LDS rows
// are padded by 16 bytes so the 16 lanes reading 16 consecutive rows at the
// same column hit distinct banks.  The epilogue rounds to bf16 and writes 4
// consecutive outputs (8 bytes) per lane.
#include "qmv_internal.h"

namespace qmv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BK = 64;             // one W4A16 group per k-step
constexpr int LDS_STRIDE = BK + 8; // bf16 elements per LDS row (144 bytes)

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// BN x BM tile, waves arranged WN x WM (WN * WM = 4).
template <int BN, int BM, int WN, int WM>
__global__ __launch_bounds__(kThreads) void gemm_w4g64_kernel(
    const uint8_t* __restrict__ Wq, const uint32_t* __restrict__ Wsz, const uint16_t* __restrict__ X,
    uint16_t* __restrict__ Y, int M, int N, int K, int vec_store) {
  static_assert(WN * WM == 4, "4 waves");
  constexpr int TN = BN / WN, TM = BM / WM;  // wave tile
  constexpr int FN = TN / 16, FM = TM / 16;  // 16x16 fragments per wave
  static_assert(FN * 16 == TN && FM * 16 == TM, "wave tile must be a multiple of 16");
  constexpr int WTASKS = BN * 2;             // 16-byte nibble chunks (32 weights) per k-step
  constexpr int WPER = (WTASKS + kThreads - 1) / kThreads;
  constexpr int XCHUNKS = BM * (BK / 8);     // 16-byte bf16 chunks per k-step
  constexpr int XPER = (XCHUNKS + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) uint16_t Ws[BN * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[BM * LDS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wm = wave / WN;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int nk = K / BK;
  const int64_t qrow = K / 2;   // nibble bytes per weight row
  const int64_t grow = K / 64;  // groups per weight row

  // global -> register staging for one k-step
  uint4 wq[WPER];
  uint32_t wsz[WPER];
  uint4 xr[XPER];
  auto load_step = [&](int ks) {
#pragma unroll
    for (int i = 0; i < WPER; ++i) {
      const int t = tid + i * kThreads;
      if (t < WTASKS) {
        const int r = t >> 1, half = t & 1;
        const int n = min(n0 + r, N - 1);
        wq[i] = *reinterpret_cast<const uint4*>(Wq + n * qrow + ks * 32 + half * 16);
        wsz[i] = Wsz[n * grow + ks];
      }
    }
#pragma unroll
    for (int i = 0; i < XPER; ++i) {
      const int t = tid + i * kThreads;
      if (t < XCHUNKS) {
        const int r = t >> 3, c = t & 7;
        const int m = m0 + r;
        xr[i] = m < M ? *reinterpret_cast<const uint4*>(X + int64_t(m) * K + ks * BK + c * 8)
                      : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int i = 0; i < WPER; ++i) {
      const int t = tid + i * kThreads;
      if (t < WTASKS) {
        const int r = t >> 1, half = t & 1;
        const float s = f16_bits_to_f32(wsz[i] & 0xFFFFu);
        const float c = -(s * f16_bits_to_f32(wsz[i] >> 16));
        const uint32_t wd[4] = {wq[i].x, wq[i].y, wq[i].z, wq[i].w};
        uint32_t o[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // byte b of wd[j] holds k = 8j + 2b (low nibble) and 8j + 2b + 1 (high nibble)
          float w[8];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (wd[j] >> (8 * b)) & 0xFFu;
            w[2 * b] = fmaf(s, static_cast<float>(byte & 15u), c);
            w[2 * b + 1] = fmaf(s, static_cast<float>(byte >> 4), c);
          }
#pragma unroll
          for (int p = 0; p < 4; ++p) o[4 * j + p] = pack_bf16x2(w[2 * p], w[2 * p + 1]);
        }
        uint4* dst = reinterpret_cast<uint4*>(Ws + r * LDS_STRIDE + half * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
      }
    }
#pragma unroll
    for (int i = 0; i < XPER; ++i) {
      const int t = tid + i * kThreads;
      if (t < XCHUNKS) {
        const int r = t >> 3, c = t & 7;
        *reinterpret_cast<uint4*>(Xs + r * LDS_STRIDE + c * 8) = xr[i];
      }
    }
  };

  f32x4 acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15;        // fragment row (weight row for A, token row for B)
  const int fk = (lane >> 4) * 8;  // this lane's 8 k values inside a 32-wide chunk

  load_step(0);
  for (int ks = 0; ks < nk; ++ks) {
    store_step();
    __syncthreads();
    if (ks + 1 < nk) load_step(ks + 1);
#pragma unroll
    for (int kc = 0; kc < BK / 32; ++kc) {
      bf16x8 a[FN], b[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(Ws + (wn * TN + i * 16 + fr) * LDS_STRIDE + kc * 32 + fk);
#pragma unroll
      for (int j = 0; j < FM; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(Xs + (wm * TM + j * 16 + fr) * LDS_STRIDE + kc * 32 + fk);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // C[n][m] fragment: lane holds n = 4*(lane/16) + e, m = lane % 16
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int n = n0 + wn * TN + i * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m0 + wm * TM + j * 16 + (lane & 15);
      if (m < M) {
        const f32x4 v = acc[i][j];
        uint16_t* dst = Y + int64_t(m) * N + n;
        if (vec_store && n + 3 < N) {  // 8-byte aligned: N % 4 == 0 and Y 8-byte aligned
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) dst[e] = static_cast<uint16_t>(pack_bf16x2(v[e], 0.f) & 0xFFFFu);
        }
      }
    }
  }
}

template <int BN, int BM, int WN, int WM>
hipError_t go(const uint8_t* W, const Planes& p, const uint16_t* X, uint16_t* Y, int M, int N, int K,
              hipStream_t s) {
  const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  const int vec = (N % 4 == 0) && (reinterpret_cast<uintptr_t>(Y) % 8 == 0);
  hipLaunchKernelGGL((gemm_w4g64_kernel<BN, BM, WN, WM>), grid, dim3(kThreads), 0, s, W,
                     reinterpret_cast<const uint32_t*>(W + p.off[1]), X, Y, M, N, K, vec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int fmt, int64_t N, int64_t K, int64_t M, const uint8_t* W, const uint16_t* X,
                       uint16_t* Y, hipStream_t s) {
  if (fmt != QMV_W4A16_G64) return hipErrorInvalidValue;
  const Planes p = planes_of(fmt, N, K);
  const int n = int(N), k = int(K), m = int(M);
  if (m <= 16) return go<64, 16, 4, 1>(W, p, X, Y, m, n, k, s);
  if (m <= 32) return go<64, 32, 4, 1>(W, p, X, Y, m, n, k, s);
  if (m <= 128) return go<64, 64, 2, 2>(W, p, X, Y, m, n, k, s);
  return go<96, 128, 2, 2>(W, p, X, Y, m, n, k, s);
}

}  // namespace qmv
