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
//     high + low is added in f32, the offset is removed with the block's
//     sum of the parts (an MFMA of A against ones; Q6K, whose sub-blocks have
//     no min, instead runs its code MFMA on top of an MFMA of A against -160,
//     which leaves sum_k (q - 32) * part), and the block scale and min are
//     applied in f32 in the same order as the dequantization formulas, so a
//     one-hot x returns the dequantized column bit for bit.
//   * Set-up: the two lanes of a high / low pair each load half of the
//     pair's activations, split them into both parts and swap the part the
//     other lane needs (one DPP move per two values).
// Work layout: a workgroup of W waves owns one 16-row tile at a time and
// strides over tiles; wave w owns KF consecutive blocks of K and keeps their
// A operands in registers for the whole launch.  The W partial
// sums of a tile meet in LDS and are added in wave order (deterministic).
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (and 16x16x16 with 4 elements):
// A[i][k] and B[k][j] sit in lane i (resp. j) + 16 * (k / 8), element k % 8;
// D[i][j] in lane j + 16 * (i / 4), element i % 4.  Any permutation of the k
// of one MFMA that A and B share leaves the product unchanged; the loaders
// below pick the one that makes each lane's weight bytes contiguous.
#include <algorithm>

#include <climits>
#include <type_traits>

#include "qmv_internal.h"

namespace qmv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// waves per workgroup: up to 8 with 8 blocks of K per wave, up to 12 with 16
template <int KF>
constexpr int kMaxWaves = KF == 8 ? 8 : 12;

struct MfmaArgs {
  const uint8_t* W;
  int64_t off1, off2, off3;  // plane offsets (bytes) from W
  const void* x;             // [nv][K]
  float* y;                  // [nv][N]
  int N, K, nv, waves;
};

// Up to kMaxSeg matrices of one format, K and vector count per launch (a
// grouped call): each segment owns a contiguous range of workgroups, sized in
// proportion to its 16-row tiles; a workgroup finds its segment once, builds
// that segment's activation operands and strides over its tiles only.  The
// table travels in the kernel arguments.
constexpr int kMaxSeg = 16;
struct MSeg {
  const uint8_t* W;
  int64_t off1, off2, off3;
  const void* x;
  float* y;
  int N;
  int b0, nb;  // first workgroup, workgroups
  int fmt;     // format (read by the mixed Q4K / Q6K kernel only)
};
constexpr int kMixM = 0;  // table format of a Q4K / Q6K mix
// The table is the kernel argument, so its size is paid by every launch:
// kernels take a table of capacity CAP = 1, 4 or 16, the smallest that holds
// the launch's segments (the batch-1 kernels measured ~0.3 us per launch
// between 16 and 4 entries).
template <int CAP>
struct MTableT {
  int first[CAP];  // first workgroup of each segment (INT_MAX past count): one wide scalar load
  MSeg s[CAP];
  int count, K, nv, waves;
};
// A single matvec with a fused epilogue (one segment): W2 != null runs
// SwiGLU, y = silu(W x) * (W2 x), W2 of the same format and shape; otherwise
// y = res + (W x + bias) with either pointer possibly null.
struct MEpi {
  const uint8_t* W2;
  const float* bias;
  const float* res;  // [nv][N]
};
struct MTableEpi {
  int first[1];
  MSeg s[1];
  int count, K, nv, waves;
  MEpi ep;
};
using MTable = MTableT<kMaxSeg>;  // built on the host, then shrunk to the launch

template <int CAP>
MTableT<CAP> shrink(const MTable& t) {  // t.count <= CAP
  MTableT<CAP> o{};
  for (int i = 0; i < CAP; ++i) {
    o.first[i] = t.first[i];
    o.s[i] = t.s[i];
  }
  o.count = t.count;
  o.K = t.K;
  o.nv = t.nv;
  o.waves = t.waves;
  return o;
}

MTableEpi with_epi(const MTable& t, const MEpi& ep) {  // t.count == 1
  MTableEpi o{};
  o.first[0] = t.first[0];
  o.s[0] = t.s[0];
  o.count = 1;
  o.K = t.K;
  o.nv = t.nv;
  o.waves = t.waves;
  o.ep = ep;
  return o;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// High (low = false) or low bf16 part of two activations, packed.
__device__ __forceinline__ uint32_t part_pair(float a, float b, bool low) {
  const float ha = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) & 0xFFFF0000u);
  const float hb = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, b) & 0xFFFF0000u);
  return pack_bf16x2(low ? a - ha : ha, low ? b - hb : hb);
}

// Both bf16 parts of two activations a, b, packed: hi = the values with
// their low 16 bits cleared (exact), lo = the rest rounded to bf16.
__device__ __forceinline__ void parts2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const uint32_t ab = __builtin_bit_cast(uint32_t, a), bb = __builtin_bit_cast(uint32_t, b);
  hi = __builtin_amdgcn_perm(bb, ab, 0x07060302u);
  lo = pack_bf16x2(a - __builtin_bit_cast(float, ab & 0xFFFF0000u), b - __builtin_bit_cast(float, bb & 0xFFFF0000u));
}

// A high / low lane pair (lanes 2i, 2i + 1: parts of one vector) each hold
// two of four activations of one operand dword pair: the even lane the first
// two (dword P0), the odd lane the last two (dword P1).  Each computes both
// parts of its own two and sends its partner the part the partner needs, so
// the pair's lanes end with (hi, hi) resp. (lo, lo) of all four in k order.
__device__ __forceinline__ void exchange_parts(float a, float b, bool low, uint32_t& p0, uint32_t& p1) {
  uint32_t hi, lo;
  parts2(a, b, hi, lo);
  // the adjacent lane's value (0 <-> 1, 2 <-> 3, ...): DPP quad_perm [1,0,3,2]
  const uint32_t got = __builtin_amdgcn_update_dpp(0, int(low ? hi : lo), 0xB1, 0xF, 0xF, false);
  p0 = low ? got : hi;
  p1 = low ? lo : got;
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

// Activations at x + off .. + 7 (f32 or f16 storage), as f32; zero unless
// `valid`.  The address must be inside x either way: the load is unconditional
// (a branch per load would keep the compiler from bounding the set-up's loads
// in flight).
template <bool XF16>
__device__ __forceinline__ void load_x8(const void* x, int64_t off, bool valid, float (&v)[8]) {
  if constexpr (XF16) {
    const u32x4 h = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = valid ? f16_bits_to_f32(h[i] & 0xFFFFu) : 0.0f;
      v[2 * i + 1] = valid ? f16_bits_to_f32(h[i] >> 16) : 0.0f;
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + off);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = valid ? a[i] : 0.0f;
      v[4 + i] = valid ? b[i] : 0.0f;
    }
  }
}

// ------------------------------------------------- per-format weight staging
//
// Per tile, each wave moves its K slice of the 16 weight rows in chunks of
// 256 k (one Q4K / Q6K super-block, four W4A16 groups, eight Q8_0 blocks):
// coalesced 16-byte global loads into registers, then into the wave's own
// LDS region, from where each lane reads its MFMA operands.  16-byte pieces
// of a row are XOR-permuted by row so that the 64 lanes' operand reads of one
// MFMA fall in distinct LDS banks.  LDS layout of a chunk (dwords):
//   codes   rows of 32 dwords (Q8_0: 64); piece p of row r at
//           32r + 4 (p ^ ((r / 2) % 8))   (Q8_0: 64r + 4 (p ^ r))
//   aux     at 512 (Q8_0: 1024): W4A16 sz and Q8_0 scales [16][4];
//           Q6K high bits [16][16] (piece p of row r at 16r + 4 (p ^ ((r / 4) % 4)))
//           and Q6K sub-block scales [16][4] at 768.
template <int FMT>
struct Stage;  // one chunk in flight, per lane
template <>
struct Stage<QMV_Q4K> { u32x4 q[2]; u32x4 meta; };
template <>
struct Stage<QMV_W4A16_G64> { u32x4 q[2]; uint32_t sz; };
template <>
struct Stage<QMV_Q8_0> { u32x4 q[4]; uint32_t sc; };
template <>
struct Stage<QMV_Q6K> { u32x4 ql[2]; u32x4 qh; uint32_t s; uint32_t d; };

template <int FMT>
constexpr int kStageDw = FMT == QMV_Q8_0 ? 1024 + 64 : FMT == QMV_Q6K ? 512 + 256 + 64 : FMT == QMV_W4A16_G64 ? 512 + 64 : 512;

__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ones8() {
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(1.0f);
  return o;
}

template <int FMT>
struct Staging {
  const MfmaArgs& a;
  int U, nsb, lane;

  // chunk of 256 k starting at fragment u, rows tile * 16 .. + 15 (clamped to
  // N - 1).  Wave-uniform chunk bases and 32-bit per-lane offsets (packed
  // matrices on this path stay below 2 GiB).  Where a chunk runs past the end
  // of a row (W4A16 / Q8_0 with K not a multiple of 256), its blocks are
  // clamped to the row's last block and never multiplied.
  __device__ __forceinline__ Stage<FMT> load(int tile, int u) const {
    Stage<FMT> st;
    const uint32_t K = a.K;
    auto row = [&](int i) { return uint32_t(min(tile * 16 + i, a.N - 1)); };
    auto ld4 = [](const uint8_t* base, uint32_t off) {
      return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
    };
    if constexpr (FMT == QMV_Q4K || FMT == QMV_Q6K) {
      const int sb = u >> 3;
      const uint8_t* qb = a.W + 128 * sb;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t off = row(8 * i + (lane >> 3)) * (K >> 1) + 16 * (lane & 7);
        if constexpr (FMT == QMV_Q4K) st.q[i] = ld4(qb, off); else st.ql[i] = ld4(qb, off);
      }
      if constexpr (FMT == QMV_Q4K) {
        st.meta = *reinterpret_cast<const u32x4*>(a.W + a.off1 + 16 * sb + row(lane & 15) * (16 * uint32_t(nsb)));
      } else {
        const uint32_t r4 = row(lane >> 2);
        st.qh = ld4(a.W + a.off1 + 64 * sb, r4 * (K >> 2) + 16 * (lane & 3));
        st.s = *reinterpret_cast<const uint32_t*>(a.W + a.off2 + 16 * sb + r4 * (K >> 4) + 4 * (lane & 3));
        st.d = *reinterpret_cast<const uint16_t*>(a.W + a.off3 + 2 * sb + row(lane & 15) * (2 * uint32_t(nsb)));
      }
    } else if constexpr (FMT == QMV_W4A16_G64) {
      const int ng = K >> 6, g0 = u >> 1;
      const bool full = g0 + 4 <= ng;  // wave-uniform
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int pc = lane & 7;
        const uint32_t rb = row(8 * i + (lane >> 3)) * (K >> 1);
        if (full) {
          st.q[i] = ld4(a.W + 32 * g0, rb + 16 * pc);
        } else {
          const int g = min(g0 + (pc >> 1), ng - 1);
          st.q[i] = ld4(a.W, rb + 32 * g + 16 * (pc & 1));
        }
      }
      st.sz = *reinterpret_cast<const uint32_t*>(a.W + a.off1 +
                                                 4 * (row(lane >> 2) * uint32_t(ng) + min(g0 + (lane & 3), ng - 1)));
    } else {  // Q8_0
      const bool full = u + 8 <= U;  // wave-uniform
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pc = lane & 15;
        const uint32_t rb = row(4 * i + (lane >> 4)) * K;
        if (full) {
          st.q[i] = ld4(a.W + 32 * u, rb + 16 * pc);
        } else {
          const int bk = min(u + (pc >> 1), U - 1);
          st.q[i] = ld4(a.W, rb + 32 * bk + 16 * (pc & 1));
        }
      }
      const uint16_t* sp = reinterpret_cast<const uint16_t*>(a.W + a.off1) + row(lane >> 2) * uint32_t(U);
      const int j = u + 2 * (lane & 3);
      st.sc = uint32_t(sp[min(j, U - 1)]) | (uint32_t(sp[min(j + 1, U - 1)]) << 16);
    }
    return st;
  }

  __device__ __forceinline__ void store(const Stage<FMT>& st, uint32_t* lds) const {
    if constexpr (FMT == QMV_Q8_0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + (lane >> 4), p = lane & 15;
        *reinterpret_cast<u32x4*>(lds + 64 * r + 4 * (p ^ r)) = st.q[i];
      }
      lds[1024 + 4 * (lane >> 2) + (lane & 3)] = st.sc;
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 8 * i + (lane >> 3), p = lane & 7;
        u32x4 v;
        if constexpr (FMT == QMV_Q6K) v = st.ql[i]; else v = st.q[i];
        *reinterpret_cast<u32x4*>(lds + 32 * r + 4 * (p ^ swz8(r))) = v;
      }
      if constexpr (FMT == QMV_W4A16_G64) {
        lds[512 + 4 * (lane >> 2) + (lane & 3)] = st.sz;
      } else if constexpr (FMT == QMV_Q6K) {
        const int r = lane >> 2, p = lane & 3;
        *reinterpret_cast<u32x4*>(lds + 512 + 16 * r + 4 * (p ^ swz4(r))) = st.qh;
        lds[768 + 4 * r + p] = st.s;
      }
    }
  }

  // acc += the chunk's contribution (fragments u .. u + 7 of this wave's
  // operands A) for vectors 2G (acc0) and 2G + 1 (acc1) of row r = lane & 15
  __device__ __forceinline__ void compute(const Stage<FMT>& st, const uint32_t* lds, const bf16x8* A, int u,
                                          float& acc0, float& acc1) const {
    const int r = lane & 15, G = lane >> 4;
    const f32x4 z = {0, 0, 0, 0};
    const bf16x8 ones = ones8();
    if constexpr (FMT == QMV_Q4K) {
      const u32x4 m = st.meta;
      const float d = f16f(m[0]), dmin = f16f(m[0] >> 16);
      const uint64_t lo = uint64_t(m[1]) | (uint64_t(m[2]) << 32);
      const uint64_t hi = uint64_t(m[2] >> 16) | (uint64_t(m[3]) << 16);
      // per super-block: sum_j sc_j (sum q x)_j and sum_j m_j (sum x)_j, then
      // d and dmin once (sc_j q and d sc_j q are exact for f16 d, so a one-hot
      // x still returns (d sc_j) q - dmin m_j bit for bit)
      float q0 = 0.0f, q1 = 0.0f, m0 = 0.0f, m1 = 0.0f;
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const uint32_t w = lds[32 * r + 4 * (f ^ swz8(r)) + G];
        const f32x4 dq = mfma32(A[f], nib8(w), z);
        const f32x4 dx = mfma32(A[f], ones, z);
        const float sc = static_cast<float>(static_cast<uint32_t>(lo >> (6 * f)) & 63u);
        const float mj = static_cast<float>(static_cast<uint32_t>(hi >> (6 * f)) & 63u);
        const float s0 = dx[0] + dx[1], s1 = dx[2] + dx[3];
        q0 = fmaf(sc, fmaf(-128.0f, s0, dq[0] + dq[1]), q0);
        q1 = fmaf(sc, fmaf(-128.0f, s1, dq[2] + dq[3]), q1);
        m0 = fmaf(mj, s0, m0);
        m1 = fmaf(mj, s1, m1);
      }
      acc0 = fmaf(-dmin, m0, fmaf(d, q0, acc0));
      acc1 = fmaf(-dmin, m1, fmaf(d, q1, acc1));
    } else if constexpr (FMT == QMV_W4A16_G64) {
      const u32x4 sz = *reinterpret_cast<const u32x4*>(lds + 512 + 4 * r);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (u + 2 * g >= U) break;
        const u32x2 w = *reinterpret_cast<const u32x2*>(lds + 32 * r + 4 * ((2 * g + (G >> 1)) ^ swz8(r)) + 2 * (G & 1));
        const f32x4 dq = mfma32(A[2 * g + 1], nib8(w[1]), mfma32(A[2 * g], nib8(w[0]), z));
        const f32x4 dx = mfma32(A[2 * g + 1], ones, mfma32(A[2 * g], ones, z));
        const float s = f16f(sz[g]), zr = f16f(sz[g] >> 16);
        const float s0 = dx[0] + dx[1], s1 = dx[2] + dx[3];
        acc0 = fmaf(s, fmaf(-zr, s0, fmaf(-128.0f, s0, dq[0] + dq[1])), acc0);
        acc1 = fmaf(s, fmaf(-zr, s1, fmaf(-128.0f, s1, dq[2] + dq[3])), acc1);
      }
    } else if constexpr (FMT == QMV_Q8_0) {
      const u32x4 sc = *reinterpret_cast<const u32x4*>(lds + 1024 + 4 * r);
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        if (u + f >= U) break;
        const u32x2 w = *reinterpret_cast<const u32x2*>(lds + 64 * r + 4 * ((2 * f + (G >> 1)) ^ r) + 2 * (G & 1));
        const f32x4 dq = mfma32(A[f], sbyte8(w[0], w[1]), z);
        const f32x4 dx = mfma32(A[f], ones, z);
        const float s = f16f(sc[f >> 1] >> (16 * (f & 1)));
        acc0 = fmaf(s, fmaf(-128.0f, dx[0] + dx[1], dq[0] + dq[1]), acc0);
        acc1 = fmaf(s, fmaf(-128.0f, dx[2] + dx[3], dq[2] + dq[3]), acc1);
      }
    } else {  // Q6K
      // lane group G takes k = 4G .. 4G + 3 of each 16-k sub-block: bytes
      // 2 (G % 2), + 1 of code word G / 2, both nibbles (k in order), with the
      // high bits of that word's even / odd codes (qh bits 4 (G / 2) + 0 / 2)
      const int g2 = G >> 1;
      const uint32_t selp = (G & 1) ? 0x07030602u : 0x05010400u;  // (even, odd, even, odd) codes of 2 bytes
      const s16x4 m160 = {-15584, -15584, -15584, -15584};  // bf16 -160 (0xC320)
      const float d = f16f(st.d);
      const u32x4 sv = *reinterpret_cast<const u32x4*>(lds + 768 + 4 * r);
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const u32x4 aw = __builtin_bit_cast(u32x4, A[f]);
        const u32x2 hw = *reinterpret_cast<const u32x2*>(lds + 512 + 16 * r + 4 * ((f >> 1) ^ swz4(r)) + 2 * (f & 1));
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint32_t qlw = lds[32 * r + 4 * (f ^ swz8(r)) + 2 * s + g2];
          const uint32_t ev = (qlw & 0x0F0F0F0Fu) | (((hw[s] >> (4 * g2)) & 0x03030303u) << 4);
          const uint32_t od = ((qlw >> 4) & 0x0F0F0F0Fu) | (((hw[s] >> (4 * g2 + 2)) & 0x03030303u) << 4);
          const uint32_t v = __builtin_amdgcn_perm(od, ev, selp);
          const u32x2 bw = {code_pair<0x04010400u>(v), code_pair<0x04030402u>(v)};
          const u32x2 aa = {aw[2 * s], aw[2 * s + 1]};
          const s16x4 a4 = __builtin_bit_cast(s16x4, aa);
          // sum_k part * (q - 32): the codes 128 + q against the parts, on top
          // of -160 times the parts' sum (one MFMA of the parts against -160)
          const f32x4 dq = mfma16(a4, __builtin_bit_cast(s16x4, bw), mfma16(a4, m160, z));
          const int j = 2 * f + s;  // sub-block within the super-block
          const float ds = d * static_cast<float>(static_cast<int8_t>((sv[j >> 2] >> (8 * (j & 3))) & 0xFFu));
          acc0 = fmaf(ds, dq[0] + dq[1], acc0);
          acc1 = fmaf(ds, dq[2] + dq[3], acc1);
        }
      }
    }
  }
};

// ------------------------------------------------------------------ kernel
//
// Per-format k order of fragment u (32 k of K), lane group G = lane >> 4:
//   Q8_0, Q4K   k = 32u + 8G + e                 (e = 0..7: the lane's 8 bytes / one nibble word)
//   W4A16       k = 64(u/2) + 16G + 8(u%2) + e    (one 8-byte read per lane serves both halves
//                                                  of the 64-k group)
//   Q6K         two 16x16x16 MFMAs, sub-block s = 0, 1:
//               k = 32u + 16s + 4G + e           (e = 0..3: two bytes of one code word, even
//                                                  and odd codes interleaved by one permute;
//                                                  elements 4s + e of the A fragment)
//
// One workgroup's share of one segment: stage is the workgroup's staging LDS
// (SD dwords per wave), red its reduction LDS.
// EPI: 0 none, 1 bias / residual (tb.ep), 2 SwiGLU with tb.ep.W2: the
// workgroup then takes each of its tiles twice, gate rows (virtual tile 2n)
// then the same up rows (2n + 1), and writes silu(gate) * up.
template <int FMT, bool XF16, int KF, int SD, int EPI = 0, class TB>
__device__ __forceinline__ void mfma_segment(const TB& tb, const MSeg& sg, uint32_t* stage, float* red) {
  constexpr int MW = kMaxWaves<KF>;
  const MfmaArgs a{sg.W, sg.off1, sg.off2, sg.off3, sg.x, sg.y, sg.N, tb.K, tb.nv, tb.waves};
  const int bid = int(blockIdx.x) - sg.b0, nblk = sg.nb;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: chunk bases in SGPRs
  const int G = lane >> 4;
  const int p = lane & 15;  // A row: part p = 2 * vector + low
  const int vec = p >> 1;
  const bool low = p & 1;
  const int K = a.K, N = a.N;
  const int U = K >> 5;
  const int u0 = wave * KF;
  const bool vec_ok = vec < a.nv;
  const int64_t xrow = int64_t(min(vec, a.nv - 1)) * K;  // address stays inside x for padding parts
  const int ntiles = (N + 15) >> 4;
  const Staging<FMT> stg{a, U, K >> 8, lane};
  MfmaArgs a2 = a;
  if constexpr (EPI == 2) a2.W = tb.ep.W2;  // same format, shape and plane offsets
  const Staging<FMT> stg2{a2, U, K >> 8, lane};

  uint32_t* lds = stage + wave * SD;

  // First weight chunk of the first tile in flight before the activations are
  // set up.  With 8 fragments per wave (one chunk of 256 k per tile) two
  // register sets take this workgroup's tiles in turn, each refilled two tiles
  // ahead as soon as its chunk is in LDS, so the next tile's loads are in
  // flight while one tile is computed; the second set's first loads go out
  // after the set-up.  A set is never copied while its loads are in flight
  // (the copy would wait for them).  With 16 fragments (two chunks per tile)
  // a second set refilled across tiles does not fit in the registers next to
  // the operands (the kernels spilled): one set is refilled with the following
  // chunk, except on a wave with a single tile (below).
  constexpr bool TWO = KF == 8;
  // this workgroup's tiles bid, bid + nblk, ... (a segment has at most as many
  // workgroups as tiles); with SwiGLU each twice (virtual tiles n = 2i, 2i + 1)
  constexpr int VT = EPI == 2 ? 2 : 1;
  const int ntl = VT * ((ntiles - bid + nblk - 1) / nblk);  // virtual tiles of this workgroup
  auto tile_of = [&](int n) { return bid + (n / VT) * nblk; };
  auto vload = [&](int n, int u) -> Stage<FMT> {
    if constexpr (EPI == 2) {
      if (n & 1) return stg2.load(tile_of(n), u);
    }
    return stg.load(tile_of(n), u);
  };
  Stage<FMT> SA = vload(0, u0), SB;

  // ---- A operands of this wave's K slice, built once (the fp16 path zeroes
  // them past K and for vectors >= nv; the f32 paths need not, see there)
  bf16x8 A[KF];
#pragma unroll
  for (int f = 0; f < KF; ++f) {
    const int u = u0 + f;
    const int uc = min(u, U - 1);
    const bool ok = vec_ok && u < U;
    if constexpr (FMT == QMV_Q6K) {  // f32 x: k = 32u + 16s + 4G + e (the code words are interleaved to match)
      // the two lanes of a high / low pair need the same 4 values of a
      // sub-block (dwords 2s, 2s + 1): each loads two and exchanges parts
      // with its partner.  No zeroing: a padding vector's A rows only reach D
      // rows that are never stored, and a wave's chunks past K are never
      // multiplied (K is a multiple of 256)
      uint32_t p[4];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x2 mine =
            *reinterpret_cast<const f32x2*>(static_cast<const float*>(a.x) + xrow + 32 * uc + 16 * s + 4 * G + 2 * low);
        exchange_parts(mine[0], mine[1], low, p[2 * s], p[2 * s + 1]);
      }
      A[f] = as_bf8(p[0], p[1], p[2], p[3]);
    } else if constexpr (!XF16) {
      // f32 x: the two lanes of a high / low pair (adjacent lanes) need the same
      // 8 values (dwords 0, 1 from the even lane's load, 2, 3 from the odd
      // lane's); each loads one half and exchanges parts with its partner,
      // halving the activation traffic.  No zeroing, as for Q6K: padding
      // vectors reach only D rows that are never stored, and fragments past K
      // are never multiplied (Q4K: K is a multiple of 256; W4A16 / Q8_0: the
      // compute loops stop at U)
      const int k0 = (FMT == QMV_W4A16_G64) ? 64 * (uc >> 1) + 16 * G + 8 * (uc & 1) : 32 * uc + 8 * G;
      const f32x4 mine = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + xrow + k0 + 4 * low);
      uint32_t p[4];
      exchange_parts(mine[0], mine[1], low, p[0], p[2]);
      exchange_parts(mine[2], mine[3], low, p[1], p[3]);
      A[f] = as_bf8(p[0], p[1], p[2], p[3]);
    } else {
      const int k0 = (FMT == QMV_W4A16_G64) ? 64 * (uc >> 1) + 16 * G + 8 * (uc & 1) : 32 * uc + 8 * G;
      float v[8];
      load_x8<XF16>(a.x, xrow + k0, ok, v);
      A[f] = as_bf8(part_pair(v[0], v[1], low), part_pair(v[2], v[3], low), part_pair(v[4], v[5], low),
                    part_pair(v[6], v[7], low));
    }
    // a scheduling fence after 8 fragments' set-up; at 16 fragments all of the
    // set-up's loads go out together (two groups of 8 were 1.7 % slower on a 1.1B
    // decode token at batch 8)
    if (KF == 8 && (f & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (TWO) {
    if (ntl > 1) SB = vload(1, u0);
  }

  int buf = 0;
  float acc0, acc1;  // vectors 2G and 2G + 1 of weight row (lane & 15)
  float gate[2];     // SwiGLU: the gate totals of this thread's outputs, until the up tile
  // the W partial sums of (virtual) tile n meet in LDS, added in wave order
  auto finish = [&](int n) {
    float* rb = red + (buf * MW + wave) * 128;
    rb[2 * lane] = acc0;
    rb[2 * lane + 1] = acc1;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int tile = tile_of(n);
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // (blockDim.x: reading it adds ~256 bytes of hidden kernel arguments)
      const int t = threadIdx.x + j * 64 * a.waves;
      if (t >= 128) break;
      const int i = t & 15;  // weight row within the tile
      const int v = t >> 4;  // vector
      const int src = 2 * (i + 16 * (v >> 1)) + (v & 1);
      float s = 0.0f;
      for (int w = 0; w < a.waves; ++w) s += red[(buf * MW + w) * 128 + src];
      const int r = tile * 16 + i;
      const int rc = min(r, N - 1);
      if constexpr (EPI == 2) {
        if ((n & 1) == 0) {
          gate[j] = s;
          continue;
        }
        s = silu_mul(gate[j], s);
      } else if constexpr (EPI == 1) {
        if (tb.ep.bias) s += tb.ep.bias[rc];
        if (tb.ep.res) s = tb.ep.res[int64_t(min(v, a.nv - 1)) * N + rc] + s;
      }
      if (v < a.nv && r < N) a.y[int64_t(v) * N + r] = s;
    }
    buf ^= 1;
  };
  if constexpr (KF == 16) {
    // a wave with two chunks and a single tile (a short, deep matrix: few
    // tiles, one per workgroup) loads both chunks at once, the second into a
    // second register set; otherwise one set is refilled as below
    const int nch = (min(KF, U - u0) + 7) >> 3;  // chunks of this wave (1 or 2)
    if (nch == 2 && ntl == 1) {
      SB = vload(0, u0 + 8);
      acc0 = acc1 = 0.0f;
      stg.store(SA, lds);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      stg.compute(SA, lds, A, u0, acc0, acc1);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // operand reads done before the next store
      stg.store(SB, lds);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      stg.compute(SB, lds, A + 8, u0 + 8, acc0, acc1);
      finish(0);
      return;
    }
  }
  if constexpr (!TWO) {
    const int nch = (min(KF, U - u0) + 7) >> 3;  // chunks of this wave (1 or 2)
    for (int n = 0;; ++n) {
      acc0 = acc1 = 0.0f;
#pragma unroll
      for (int c = 0; c < KF / 8; ++c) {
        if (c >= nch) break;
        stg.store(SA, lds);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const Stage<FMT> cur = SA;
        // next chunk: the following one of this tile, else the first of the next tile
        if (c + 1 < nch) SA = vload(n, u0 + 8 * (c + 1));
        else if (n + 1 < ntl) SA = vload(n + 1, u0);
        stg.compute(cur, lds, A + 8 * c, u0 + 8 * c, acc0, acc1);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // operand reads done before the next store
      }
      finish(n);
      if (n + 1 >= ntl) return;
    }
  } else {
    // tile number n of this workgroup from set S, which then takes tile n + 2
    auto run = [&](Stage<FMT>& S, int n) {
      acc0 = acc1 = 0.0f;
      stg.store(S, lds);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const Stage<FMT> cur = S;  // its loads are done: a plain copy
      if (n + 2 < ntl) S = vload(n + 2, u0);
      stg.compute(cur, lds, A, u0, acc0, acc1);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // operand reads done before the next store
      finish(n);
    };
    for (int n = 0;; n += 2) {
      run(SA, n);
      if (n + 1 >= ntl) return;
      run(SB, n + 1);
      if (n + 2 >= ntl) return;
    }
  }
}

// FMT = kMixM: a table of Q4K and Q6K segments, each workgroup taking its
// segment's format path (a workgroup-uniform branch).
template <int FMT, bool XF16, int KF, int CAP>
__global__ __launch_bounds__(64 * kMaxWaves<KF>) void matvec_mfma_kernel(const MTableT<CAP> tb) {
  constexpr int MW = kMaxWaves<KF>;
  constexpr int SD = FMT == kMixM ? kStageDw<QMV_Q6K> : kStageDw<FMT>;
  static_assert(kStageDw<QMV_Q4K> <= kStageDw<QMV_Q6K>, "mixed staging size");
  __shared__ uint32_t stage_lds[MW * SD];
  __shared__ f32x4 red_raw[2][MW][32];  // [buffer][wave][lane pair] -> 2 x float2
  float* red = reinterpret_cast<float*>(red_raw);
  int si = 0;  // this workgroup's segment: a count over the first-workgroup array
#pragma unroll
  for (int i = 1; i < CAP; ++i) si += int(blockIdx.x) >= tb.first[i] ? 1 : 0;
  const MSeg& sg = tb.s[si];
  if constexpr (FMT == kMixM) {
    if (sg.fmt == QMV_Q6K) mfma_segment<QMV_Q6K, false, KF, SD>(tb, sg, stage_lds, red);
    else mfma_segment<QMV_Q4K, false, KF, SD>(tb, sg, stage_lds, red);
  } else {
    mfma_segment<FMT, XF16, KF, SD>(tb, sg, stage_lds, red);
  }
}

// One matvec with a fused epilogue (EPI 1: bias / residual, 2: SwiGLU).
template <int FMT, bool XF16, int KF, int EPI>
__global__ __launch_bounds__(64 * kMaxWaves<KF>) void matvec_mfma_epi_kernel(const MTableEpi tb) {
  constexpr int MW = kMaxWaves<KF>;
  __shared__ uint32_t stage_lds[MW * kStageDw<FMT>];
  __shared__ f32x4 red_raw[2][MW][32];
  mfma_segment<FMT, XF16, KF, kStageDw<FMT>, EPI>(tb, tb.s[0], stage_lds, reinterpret_cast<float*>(red_raw));
}

int blocks_override() {
  static const int v = [] {
    return ab_switch("QMV_MFMA_BLOCKS", 0);  // A/B tuning only: workgroups per launch
  }();
  return v;
}

// Workgroups: up to 256 per launch, one per CU, or 512 for Q6K (tuning
// override above), split over the segments in proportion to their tiles, at
// least one and at most one per tile.  Every wave builds its activation
// operands once per launch (about 340 vector instructions per wave for Q4K,
// against about 165 per tile), so fewer workgroups that each take more tiles,
// with the next tile's weights in flight, do less work in all (measured on
// MI355X, one 1.1B decode step at batch 8: 128 / 192 / 256 / 384 / 512
// workgroups: 0.937 / 0.831 / 0.794 / 0.832 / 0.828 ms; the grouped Q4K
// gate+up 11.0 -> 8.6 us).  Q6K launches take 512: with one register set its
// tiles ran back to back and the 32000 x 2048 head took 22.1 us at 512 and 25.8
// at 256; with two sets the 1.1B step is the same at 256 and 512 (0.692 ms).
template <int FMT, bool XF16, int KF>
hipError_t go(MTable& t, hipStream_t s, const MEpi* ep = nullptr) {
  int64_t tiles[kMaxSeg], total = 0;
  for (int i = 0; i < t.count; ++i) {
    tiles[i] = (t.s[i].N + 15) / 16;
    total += tiles[i];
  }
  int64_t budget = blocks_override();
  if (budget <= 0) budget = FMT == QMV_Q6K ? 512 : 256;
  if (budget > total) budget = total;
  int b = 0;
  for (int i = 0; i < t.count; ++i) {
    const int64_t share = (budget * tiles[i] + total - 1) / total;
    t.s[i].b0 = b;
    t.s[i].nb = int(std::max<int64_t>(1, std::min(tiles[i], share)));
    b += t.s[i].nb;
  }
  for (int i = 0; i < kMaxSeg; ++i) t.first[i] = i < t.count ? t.s[i].b0 : INT_MAX;  // INT_MAX: never selected
  const dim3 grid(b), block(64 * t.waves);
  if constexpr (FMT != kMixM) {
    if (ep) {
      if (ep->W2)
        hipLaunchKernelGGL((matvec_mfma_epi_kernel<FMT, XF16, KF, 2>), grid, block, 0, s, with_epi(t, *ep));
      else
        hipLaunchKernelGGL((matvec_mfma_epi_kernel<FMT, XF16, KF, 1>), grid, block, 0, s, with_epi(t, *ep));
      return hipGetLastError();
    }
  }
  if (t.count == 1 && FMT != kMixM)
    hipLaunchKernelGGL((matvec_mfma_kernel<FMT, XF16, KF, 1>), grid, block, 0, s, shrink<1>(t));
  else if (t.count <= 4)
    hipLaunchKernelGGL((matvec_mfma_kernel<FMT, XF16, KF, 4>), grid, block, 0, s, shrink<4>(t));
  else
    hipLaunchKernelGGL((matvec_mfma_kernel<FMT, XF16, KF, kMaxSeg>), grid, block, 0, s, t);
  return hipGetLastError();
}

template <int FMT, bool XF16>
bool pick_kf(MTable& t, hipStream_t s, hipError_t* err, const MEpi* ep = nullptr) {
  const int U = t.K / 32;
  // fragments per wave, a multiple of 8 (whole Q4K / Q6K super-blocks, W4A16
  // group pairs): 8 up to K = 2048 (at most 8 waves), else 16 (at most 12 waves,
  // K <= 6144)
  const int kf = U <= 8 * kMaxWaves<8> ? 8 : 16;
  t.waves = (U + kf - 1) / kf;
  if (t.waves > (kf == 8 ? kMaxWaves<8> : kMaxWaves<16>)) return false;
  *err = kf == 8 ? go<FMT, XF16, 8>(t, s, ep) : go<FMT, XF16, 16>(t, s, ep);
  return true;
}

bool launch_table(int fmt, MTable& t, int x_dtype, hipStream_t s, hipError_t* err, const MEpi* ep = nullptr) {
  if (x_dtype == QMV_Q8X) return false;  // 8-bit activations run on the general kernel
  const bool f16 = (x_dtype == QMV_F16);
  switch (fmt) {
    case QMV_Q8_0: return pick_kf<QMV_Q8_0, false>(t, s, err, ep);
    case QMV_W4A16_G64:
      return f16 ? pick_kf<QMV_W4A16_G64, true>(t, s, err, ep) : pick_kf<QMV_W4A16_G64, false>(t, s, err, ep);
    case QMV_Q4K: return pick_kf<QMV_Q4K, false>(t, s, err, ep);
    case QMV_Q6K: return pick_kf<QMV_Q6K, false>(t, s, err, ep);
    case kMixM: return ep ? false : pick_kf<kMixM, false>(t, s, err);
    default: return false;
  }
}

// Formats this kernel takes (the others run on the general kernel).
bool has_kernel(int fmt) {
  return fmt == QMV_Q8_0 || fmt == QMV_W4A16_G64 || fmt == QMV_Q4K || fmt == QMV_Q6K;
}

bool fits(int fmt, int64_t N, int64_t K) {
  // the kernel addresses planes with 32-bit offsets; K up to 12 waves x 16 blocks
  return planes_of(fmt, N, K).total < (int64_t(1) << 31) && K / 32 <= 12 * 16;
}

}  // namespace

// 2..8 vectors on the matrix cores.  Returns false (nothing launched) for
// shapes outside this kernel's range (K > 6144, packed matrix >= 2 GiB).
bool launch_matvec_mfma(int fmt, int64_t N, int64_t K, int nv, const uint8_t* W, const void* x, int x_dtype,
                        float* y, hipStream_t s, hipError_t* err) {
  return launch_matvec_mfma_epi(fmt, N, K, nv, W, nullptr, x, x_dtype, y, nullptr, nullptr, s, err);
}

// The same with a fused epilogue: W2 != null runs SwiGLU (y = silu(W x) *
// (W2 x)), otherwise y = res + (W x + bias) (bias [N], res [nv][N], either
// null).  All null: the plain kernel.
bool launch_matvec_mfma_epi(int fmt, int64_t N, int64_t K, int nv, const uint8_t* W, const uint8_t* W2,
                            const void* x, int x_dtype, float* y, const float* bias, const float* res,
                            hipStream_t s, hipError_t* err) {
  if (!has_kernel(fmt) || !fits(fmt, N, K)) return false;
  const Planes p = planes_of(fmt, N, K);
  MTable t{};
  t.count = 1;
  t.K = int(K);
  t.nv = nv;
  t.s[0] = MSeg{W, p.off[1], p.off[2], p.off[3], x, y, int(N), 0, 0, fmt};
  if (!W2 && !bias && !res) return launch_table(fmt, t, x_dtype, s, err);
  const MEpi ep{W2, bias, res};
  return launch_table(fmt, t, x_dtype, s, err, &ep);
}

// Several matvecs of one K and batch (>= 2) on the matrix cores: per chunk of
// up to 8 vectors, one launch per kMaxSeg items of one format (items of
// different formats run in separate launch series; Q4K with Q6K share the
// mixed kernel).  An item's format is its own fmt field, or `fmt` where that
// is 0.  Returns false (nothing launched) when some item is outside the
// kernel's range.
bool launch_matvec_grouped_mfma(int fmt, int64_t K, int64_t batch, int count, const qmv_matvec_item* items,
                                int x_dtype, hipStream_t s, hipError_t* err) {
  if (x_dtype == QMV_Q8X) return false;  // 8-bit activations run on the general kernel
  auto eff = [&](int i) { return items[i].fmt ? items[i].fmt : fmt; };
  for (int i = 0; i < count; ++i)  // decided before anything is launched
    if (!has_kernel(eff(i)) || !fits(eff(i), items[i].N, K)) return false;
  const int64_t xel = (x_dtype == QMV_F16) ? 2 : 4;
  auto run = [&](int tfmt, const int* idx, int n) {
    for (int64_t b0 = 0; b0 < batch; b0 += 8) {
      const int nv = int(batch - b0 < 8 ? batch - b0 : 8);
      for (int i0 = 0; i0 < n; i0 += kMaxSeg) {
        MTable t{};
        t.K = int(K);
        t.nv = nv;
        t.count = n - i0 < kMaxSeg ? n - i0 : kMaxSeg;
        for (int j = 0; j < t.count; ++j) {
          const int i = idx[i0 + j];
          const qmv_matvec_item& it = items[i];
          const Planes p = planes_of(eff(i), it.N, K);
          t.s[j] = MSeg{static_cast<const uint8_t*>(it.W), p.off[1], p.off[2], p.off[3],
                        static_cast<const uint8_t*>(it.x) + b0 * K * xel, static_cast<float*>(it.y) + b0 * it.N,
                        int(it.N), 0, 0, eff(i)};
        }
        if (!launch_table(tfmt, t, x_dtype, s, err)) return false;
        if (*err != hipSuccess) return true;
      }
    }
    return true;
  };
  constexpr int kMaxItems = 4096;  // host-side index scratch (the API caps count below this)
  int idx[kMaxItems];
  bool same = true, kquant = true;
  for (int i = 0; i < count; ++i) {
    same = same && eff(i) == eff(0);
    kquant = kquant && (eff(i) == QMV_Q4K || eff(i) == QMV_Q6K);
  }
  if (same || kquant) {
    for (int i = 0; i < count; ++i) idx[i] = i;
    return run(same ? eff(0) : kMixM, idx, count);
  }
  for (int f = 1; f <= kNumFormats; ++f) {
    int n = 0;
    for (int i = 0; i < count; ++i)
      if (eff(i) == f) idx[n++] = i;
    if (n == 0) continue;
    if (!run(f, idx, n)) return false;
    if (*err != hipSuccess) return true;
  }
  return true;
}

}  // namespace qmv
