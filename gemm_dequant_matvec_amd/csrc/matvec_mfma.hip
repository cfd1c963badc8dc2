// Decode matvec for 2..8 activation vectors on the bf16 matrix cores.
//
// The pages' batched decode decodes each weight once and uses it against
// every activation vector in flight (aot-llm README, batched prompt notes);
// the scale / min is applied per block, outside the integer inner product.
// With 8 vectors that inner product is a small dense contraction, so here it
// runs on MFMA instead of one f32 FMA per weight and vector.
//
// One MFMA per block of 16 weight rows:
//   * B operand: the block's integer codes, exact in bf16 as 128 + q (bits
//     0x4300 | q; Q8_0 codes go through (q + 128) as an unsigned byte).
//   * A operand: 16 "parts" = 8 vectors x {high, low}: high = the f32 value
//     with its low 16 bits cleared (exact in bf16), low = the rest, rounded to
//     bf16 (|error| <= 2^-16 |x|).  No padding rows at batch 8.
//   * D (16 x 16, f32): per weight row and part, sum_k (128 + q) * part.
//     high + low is added in f32, the 128 offset is removed with the block's
//     sum of x (one MFMA of A against ones, done once per launch), and the
//     block scale and min are applied in f32 in the same order as the
//     dequantization formulas, so a one-hot x returns the dequantized column
//     bit for bit.
// Work layout: a workgroup of W waves owns one 16-row tile at a time and
// strides over tiles; wave w owns KF consecutive blocks of K and keeps their
// A operands and block sums in registers for the whole launch.  The W partial
// sums of a tile meet in LDS and are added in wave order (deterministic).
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (and 16x16x16 with 4 elements):
// A[i][k] and B[k][j] sit in lane i (resp. j) + 16 * (k / 8), element k % 8;
// D[i][j] in lane j + 16 * (i / 4), element i % 4.  Any permutation of the k
// of one MFMA that A and B share leaves the product unchanged; the loaders
// below pick the one that makes each lane's weight bytes contiguous.
#include <cstdlib>

#include "qmv_internal.h"

namespace qmv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxWaves = 8;

struct MfmaArgs {
  const uint8_t* W;
  int64_t off1, off2, off3;  // plane offsets (bytes) from W
  const void* x;             // [nv][K]
  float* y;                  // [nv][N]
  int N, K, nv, waves;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// High or low bf16 part of two activations, packed.
__device__ __forceinline__ uint32_t part_pair(float a, float b, bool low) {
  const float ha = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) & 0xFFFF0000u);
  const float hb = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, b) & 0xFFFF0000u);
  return pack_bf16x2(low ? a - ha : ha, low ? b - hb : hb);
}

__device__ __forceinline__ bf16x8 as_bf8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

// bytes c0, c1 of t as (128 + byte) bf16 pair: [t.c0, 0x43, t.c1, 0x43]
template <uint32_t SEL>
__device__ __forceinline__ uint32_t code_pair(uint32_t t) {
  return __builtin_amdgcn_perm(0x43434343u, t, SEL);
}

// 8 nibbles (byte m = q[2m] | q[2m+1] << 4, k in order) -> 8 bf16 codes 128 + q.
__device__ __forceinline__ bf16x8 nib8(uint32_t w) {
  const uint32_t ev = w & 0x0F0F0F0Fu;
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t lo = __builtin_amdgcn_perm(od, ev, 0x05010400u);  // q0 q1 q2 q3
  const uint32_t hi = __builtin_amdgcn_perm(od, ev, 0x07030602u);  // q4 q5 q6 q7
  return as_bf8(code_pair<0x04010400u>(lo), code_pair<0x04030402u>(lo), code_pair<0x04010400u>(hi),
                code_pair<0x04030402u>(hi));
}

// 8 int8 codes (two words, k in order) -> 8 bf16 codes q + 128 (exact: 0..255).
__device__ __forceinline__ bf16x8 sbyte8(uint32_t w0, uint32_t w1) {
  const uint32_t a = w0 ^ 0x80808080u, b = w1 ^ 0x80808080u;
  auto f = [](uint32_t v, int c) { return static_cast<float>((v >> (8 * c)) & 0xFFu); };
  return as_bf8(pack_bf16x2(f(a, 0), f(a, 1)), pack_bf16x2(f(a, 2), f(a, 3)), pack_bf16x2(f(b, 0), f(b, 1)),
                pack_bf16x2(f(b, 2), f(b, 3)));
}

__device__ __forceinline__ float f16f(uint32_t bits) { return f16_bits_to_f32(bits & 0xFFFFu); }

// Activations of vector `vec` at k = k0 .. k0 + 7 (f32 or f16 storage), as f32.
template <bool XF16>
__device__ __forceinline__ void load_x8(const void* x, int64_t off, bool valid, float (&v)[8]) {
  if constexpr (XF16) {
    u32x4 h = {0, 0, 0, 0};
    if (valid) h = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = f16_bits_to_f32(h[i] & 0xFFFFu);
      v[2 * i + 1] = f16_bits_to_f32(h[i] >> 16);
    }
  } else {
    f32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (valid) {
      const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + off);
      a = p[0];
      b = p[1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// ------------------------------------------------- per-format weight chunks
//
// A chunk is the weight data of CF<FMT> fragments of one row for one lane:
// 8 (one Q4K super-block, four W4A16 groups, eight Q8_0 blocks) or 4 (half a
// Q6K super-block, whose codes, high bits and scales take twice the registers).
template <int FMT>
constexpr int CF = (FMT == QMV_Q6K) ? 4 : 8;
template <int FMT>
struct Chunk;
template <>
struct Chunk<QMV_Q4K> { uint32_t q[8]; u32x4 meta; };
template <>
struct Chunk<QMV_W4A16_G64> { u32x2 q[4]; uint32_t sz[4]; };
template <>
struct Chunk<QMV_Q8_0> { u32x2 q[8]; uint32_t sc[8]; };
template <>
struct Chunk<QMV_Q6K> { uint32_t ql[4][2]; u32x2 qh[4]; u32x2 s; uint32_t d; };

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const s16x4& a, const s16x4& b) {
  const f32x4 z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, z, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ones8() {
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(1.0f);
  return o;
}

// One 16-row tile seen from one lane: its weight row and plane addressing.
template <int FMT>
struct Tile {
  const MfmaArgs& a;
  int64_t row;
  const uint8_t* qrow;
  int U, nsb, G;

  // weights of fragments u .. u + 7 (clamped into the row; fragments past K are
  // never multiplied)
  __device__ __forceinline__ Chunk<FMT> load(int u) const {
    Chunk<FMT> c;
    if constexpr (FMT == QMV_Q4K) {
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int uu = min(u + f, U - 1);
        c.q[f] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(qrow + 16 * uu + 4 * G));
      }
      c.meta = reinterpret_cast<const u32x4*>(a.W + a.off1)[row * nsb + (u >> 3)];
    } else if constexpr (FMT == QMV_W4A16_G64) {
      const int ng = a.K >> 6;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gi = min((u >> 1) + g, ng - 1);
        c.q[g] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(qrow + 32 * gi + 8 * G));
        c.sz[g] = reinterpret_cast<const uint32_t*>(a.W + a.off1)[row * ng + gi];
      }
    } else if constexpr (FMT == QMV_Q8_0) {
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int uu = min(u + f, U - 1);
        c.q[f] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(qrow + 32 * uu + 8 * G));
        c.sc[f] = reinterpret_cast<const uint16_t*>(a.W + a.off1)[row * U + uu];
      }
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int uu = min(u + f, U - 1);
        const uint32_t* w = reinterpret_cast<const uint32_t*>(qrow + 16 * uu);
        c.ql[f][0] = __builtin_nontemporal_load(w + (G >> 1));
        c.ql[f][1] = __builtin_nontemporal_load(w + 2 + (G >> 1));
        c.qh[f] = reinterpret_cast<const u32x2*>(a.W + a.off1)[row * U + uu];
      }
      // 8 int8 scales: sub-blocks 2u .. 2u + 7 (u is a multiple of 4)
      c.s = reinterpret_cast<const u32x2*>(a.W + a.off2)[(row * U + u) >> 2];
      c.d = reinterpret_cast<const uint16_t*>(a.W + a.off3)[row * nsb + (u >> 3)];
    }
    return c;
  }

  // acc += this chunk's contribution for vectors 2G (acc0) and 2G + 1 (acc1)
  __device__ __forceinline__ void compute(const Chunk<FMT>& c, const bf16x8* A, int u, float& acc0,
                                          float& acc1) const {
    const f32x4 z = {0, 0, 0, 0};
    const bf16x8 ones = ones8();
    if constexpr (FMT == QMV_Q4K) {
      const float d = f16f(c.meta[0]), dmin = f16f(c.meta[0] >> 16);
      const uint64_t lo = uint64_t(c.meta[1]) | (uint64_t(c.meta[2]) << 32);
      const uint64_t hi = uint64_t(c.meta[2] >> 16) | (uint64_t(c.meta[3]) << 16);
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        if (u + f >= U) break;
        const f32x4 dq = mfma32(A[f], nib8(c.q[f]), z);
        const f32x4 dx = mfma32(A[f], ones, z);
        const float ds = d * static_cast<float>(static_cast<uint32_t>(lo >> (6 * f)) & 63u);
        const float dm = dmin * static_cast<float>(static_cast<uint32_t>(hi >> (6 * f)) & 63u);
        const float s0 = dx[0] + dx[1], s1 = dx[2] + dx[3];
        acc0 = fmaf(-dm, s0, fmaf(ds, fmaf(-128.0f, s0, dq[0] + dq[1]), acc0));
        acc1 = fmaf(-dm, s1, fmaf(ds, fmaf(-128.0f, s1, dq[2] + dq[3]), acc1));
      }
    } else if constexpr (FMT == QMV_W4A16_G64) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (u + 2 * g >= U) break;
        const f32x4 dq = mfma32(A[2 * g + 1], nib8(c.q[g][1]), mfma32(A[2 * g], nib8(c.q[g][0]), z));
        const f32x4 dx = mfma32(A[2 * g + 1], ones, mfma32(A[2 * g], ones, z));
        const float s = f16f(c.sz[g]), zr = f16f(c.sz[g] >> 16);
        const float s0 = dx[0] + dx[1], s1 = dx[2] + dx[3];
        acc0 = fmaf(s, fmaf(-zr, s0, fmaf(-128.0f, s0, dq[0] + dq[1])), acc0);
        acc1 = fmaf(s, fmaf(-zr, s1, fmaf(-128.0f, s1, dq[2] + dq[3])), acc1);
      }
    } else if constexpr (FMT == QMV_Q8_0) {
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        if (u + f >= U) break;
        const f32x4 dq = mfma32(A[f], sbyte8(c.q[f][0], c.q[f][1]), z);
        const f32x4 dx = mfma32(A[f], ones, z);
        const float s = f16f(c.sc[f]);
        acc0 = fmaf(s, fmaf(-128.0f, dx[0] + dx[1], dq[0] + dq[1]), acc0);
        acc1 = fmaf(s, fmaf(-128.0f, dx[2] + dx[3], dq[2] + dq[3]), acc1);
      }
    } else {
      const int sh_q = 4 * (G & 1);
      const int sh_h = 4 * (G >> 1) + 2 * (G & 1);
      const s16x4 ones4 = {0x3F80, 0x3F80, 0x3F80, 0x3F80};
      const float d = f16f(c.d);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (u + f >= U) break;
        const u32x4 aw = __builtin_bit_cast(u32x4, A[f]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint32_t v = ((c.ql[f][s] >> sh_q) & 0x0F0F0F0Fu) | (((c.qh[f][s] >> sh_h) & 0x03030303u) << 4);
          const u32x2 bw = {code_pair<0x04010400u>(v), code_pair<0x04030402u>(v)};
          const u32x2 aa = {aw[2 * s], aw[2 * s + 1]};
          const s16x4 a4 = __builtin_bit_cast(s16x4, aa);
          const f32x4 dq = mfma16(a4, __builtin_bit_cast(s16x4, bw));
          const f32x4 dx = mfma16(a4, ones4);
          const int j = 2 * f + s;  // sub-block within the chunk
          const float sc = static_cast<float>(static_cast<int8_t>((c.s[j >> 2] >> (8 * (j & 3))) & 0xFFu));
          const float ds = d * sc;
          acc0 = fmaf(ds, fmaf(-160.0f, dx[0] + dx[1], dq[0] + dq[1]), acc0);
          acc1 = fmaf(ds, fmaf(-160.0f, dx[2] + dx[3], dq[2] + dq[3]), acc1);
        }
      }
    }
  }
};

// ------------------------------------------------------------------ kernel
//
// Per-format k order of fragment u (32 k of K), lane group G = lane >> 4:
//   Q8_0, Q4K   k = 32u + 8G + e                 (e = 0..7: the lane's 8 bytes / one nibble word)
//   W4A16       k = 64(u/2) + 16G + 8(u%2) + e    (one 8-byte load per lane serves both halves
//                                                  of the 64-k group)
//   Q6K         two 16x16x16 MFMAs, sub-block s = 0, 1:
//               k = 32u + 16s + 8(G/2) + 2e + G%2  (e = 0..3: one byte lane of one 6-bit code
//                                                  word; elements 4s + e of the A fragment)
template <int FMT, bool XF16, int KF>
__global__ __launch_bounds__(64 * kMaxWaves) void matvec_mfma_kernel(const MfmaArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = lane >> 4;
  const int p = lane & 15;  // A row: part p = 2 * vector + low
  const int vec = p >> 1;
  const bool low = p & 1;
  const int K = a.K, N = a.N;
  const int U = K >> 5;
  const int u0 = wave * KF;
  const bool vec_ok = vec < a.nv;
  const int64_t xrow = int64_t(min(vec, a.nv - 1)) * K;  // address stays inside x for padding parts

  // ---- A operands of this wave's K slice, built once (zero past K and for
  // vectors >= nv, so those fragments and parts contribute nothing)
  bf16x8 A[KF];
#pragma unroll
  for (int f = 0; f < KF; ++f) {
    const int u = u0 + f;
    const bool ok = vec_ok && u < U;
    float v[8];
    if constexpr (FMT == QMV_Q6K) {  // f32 x only: k = 32u + 16s + 8(G/2) + (G%2) + 2e
      const float* xp = static_cast<const float*>(a.x) + xrow + 32 * min(u, U - 1) + 8 * (G >> 1) + (G & 1);
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * s + e] = ok ? xp[16 * s + 2 * e] : 0.0f;
    } else {
      const int uc = min(u, U - 1);
      const int k0 = (FMT == QMV_W4A16_G64) ? 64 * (uc >> 1) + 16 * G + 8 * (uc & 1) : 32 * uc + 8 * G;
      load_x8<XF16>(a.x, xrow + k0, ok, v);
    }
    A[f] = as_bf8(part_pair(v[0], v[1], low), part_pair(v[2], v[3], low), part_pair(v[4], v[5], low),
                  part_pair(v[6], v[7], low));
    // at most 8 fragments' raw activations in flight (register peak of the set-up)
    if ((f & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
  __shared__ f32x4 red_raw[2][kMaxWaves][32];  // [buffer][wave][lane pair] -> 2 x float2
  float* red = reinterpret_cast<float*>(red_raw);
  const int ntiles = (N + 15) >> 4;
  const int64_t rowbytes_q = (FMT == QMV_Q8_0) ? K : (K >> 1);
  const int nsb = K >> 8;  // super-blocks per row (Q4K, Q6K)
  int buf = 0;

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t row = min(tile * 16 + p, N - 1);  // B column j = lane & 15 = weight row
    const uint8_t* qrow = a.W + row * rowbytes_q;
    float acc0 = 0.0f, acc1 = 0.0f;  // vectors 2G and 2G + 1 of weight row (lane & 15)
    const Tile<FMT> t{a, row, qrow, U, nsb, G};
    // two-stage pipeline over chunks: the next chunk's weights are in flight
    // while the current one is multiplied
    // (single stage where two chunks would not fit in registers next to 24 A
    // operands: Q6K and Q8_0 at K > 2048)
    constexpr int C = CF<FMT>;
    constexpr bool PIPE = !(KF > 8 && (FMT == QMV_Q6K || FMT == QMV_Q8_0));
    Chunk<FMT> cur = t.load(u0);
#pragma unroll
    for (int c = 0; c < KF; c += C) {
      if (u0 + c >= U) break;
      if constexpr (PIPE) {
        Chunk<FMT> nxt;
        if (c + C < KF && u0 + c + C < U) nxt = t.load(u0 + c + C);
        __builtin_amdgcn_sched_barrier(0);
        t.compute(cur, A + c, u0 + c, acc0, acc1);
        cur = nxt;
      } else {
        if (c > 0) cur = t.load(u0 + c);
        t.compute(cur, A + c, u0 + c, acc0, acc1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- the W partial sums of this tile meet in LDS, added in wave order
    float* rb = red + (buf * kMaxWaves + wave) * 128;
    rb[2 * lane] = acc0;
    rb[2 * lane + 1] = acc1;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int t = threadIdx.x; t < 128; t += blockDim.x) {
      const int i = t & 15;  // weight row within the tile
      const int v = t >> 4;  // vector
      const int src = 2 * (i + 16 * (v >> 1)) + (v & 1);
      float s = 0.0f;
      for (int w = 0; w < a.waves; ++w) s += red[(buf * kMaxWaves + w) * 128 + src];
      const int r = tile * 16 + i;
      if (v < a.nv && r < N) a.y[int64_t(v) * N + r] = s;
    }
    buf ^= 1;
  }
}

int blocks_override() {
  static const int v = [] {
    const char* e = getenv("QMV_MFMA_BLOCKS");  // A/B tuning only: workgroups per launch
    return e ? atoi(e) : 0;
  }();
  return v;
}

template <int FMT, bool XF16, int KF>
hipError_t go(const MfmaArgs& a, hipStream_t s) {
  const int ntiles = (a.N + 15) / 16;
  int blocks = blocks_override();
  if (blocks <= 0) blocks = 512;
  if (blocks > ntiles) blocks = ntiles;
  hipLaunchKernelGGL((matvec_mfma_kernel<FMT, XF16, KF>), dim3(blocks), dim3(64 * a.waves), 0, s, a);
  return hipGetLastError();
}

template <int FMT, bool XF16>
bool pick_kf(MfmaArgs& a, hipStream_t s, hipError_t* err) {
  const int U = a.K / 32;
  // fragments per wave, a multiple of 8 (whole Q4K / Q6K super-blocks, W4A16
  // group pairs): 8 up to K = 2048, else 24 (K <= 6144), at most 8 waves
  const int kf = U <= 8 * kMaxWaves ? 8 : 24;
  a.waves = (U + kf - 1) / kf;
  if (a.waves > kMaxWaves) return false;
  *err = kf == 8 ? go<FMT, XF16, 8>(a, s) : go<FMT, XF16, 24>(a, s);
  return true;
}

}  // namespace

// 2..8 vectors on the matrix cores.  Returns false (nothing launched) for
// shapes outside this kernel's range (K > 6144).
bool launch_matvec_mfma(int fmt, int64_t N, int64_t K, int nv, const uint8_t* W, const void* x, int x_dtype,
                        float* y, hipStream_t s, hipError_t* err) {
  const Planes p = planes_of(fmt, N, K);
  MfmaArgs a{W, p.off[1], p.off[2], p.off[3], x, y, int(N), int(K), nv, 0};
  const bool f16 = (x_dtype == QMV_F16);
  switch (fmt) {
    case QMV_Q8_0: return pick_kf<QMV_Q8_0, false>(a, s, err);
    case QMV_W4A16_G64:
      return f16 ? pick_kf<QMV_W4A16_G64, true>(a, s, err) : pick_kf<QMV_W4A16_G64, false>(a, s, err);
    case QMV_Q4K: return pick_kf<QMV_Q4K, false>(a, s, err);
    case QMV_Q6K: return pick_kf<QMV_Q6K, false>(a, s, err);
    default: return false;
  }
}

}  // namespace qmv
