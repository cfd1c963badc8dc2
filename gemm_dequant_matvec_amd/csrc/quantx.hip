// qmv_quantize_x: f32 activations -> 8-bit blocks for the integer-dot matvec.
//
// The pages' CPU decode path quantizes the activation vector once per matmul
// and takes integer dot products (aot-llm README, How it works).  One thread
// per block of 32 activations: the absolute maximum, d = amax / 127 and
// id = 127 / amax (correctly rounded f32 divisions; both 0 when amax < 2^-120),
// codes rint(x * id) clamped to +-127 (round half to even), 32 code bytes and
// one f32 scale out.
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int kThreads = 256;

__global__ void quantize_x_kernel(const float* __restrict__ x, uint8_t* __restrict__ xq, int64_t K,
                                  int64_t blocks, int64_t rec) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= blocks) return;
  const int64_t per = K / 32;
  const int64_t b = t / per, j = t - b * per;
  const float4* src = reinterpret_cast<const float4*>(x + b * K + 32 * j);
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 f = src[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // below 2^-120, 127 / amax could overflow: such a block is all zeros
  const bool live = amax >= 0x1p-120f;
  const float d = live ? amax / 127.0f : 0.0f;
  const float id = live ? 127.0f / amax : 0.0f;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float qf = fminf(fmaxf(rintf(v[4 * i + c] * id), -127.0f), 127.0f);
      word |= (uint32_t(int32_t(qf)) & 0xFFu) << (8 * c);
    }
    w[i] = word;
  }
  uint8_t* dst = xq + b * rec;
  uint4* q = reinterpret_cast<uint4*>(dst + 32 * j);
  q[0] = make_uint4(w[0], w[1], w[2], w[3]);
  q[1] = make_uint4(w[4], w[5], w[6], w[7]);
  reinterpret_cast<float*>(dst + K)[j] = d;
}

}  // namespace

int64_t q8x_record_bytes(int64_t K) { return (K + K / 8 + 15) / 16 * 16; }

hipError_t launch_quantize_x(int64_t K, int64_t batch, const float* x, uint8_t* xq, hipStream_t s) {
  const int64_t blocks = batch * (K / 32);
  const dim3 grid(static_cast<unsigned>((blocks + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(quantize_x_kernel, grid, dim3(kThreads), 0, s, x, xq, K, blocks, q8x_record_bytes(K));
  return hipGetLastError();
}

}  // namespace qmv
