// Decode matvec for one or two activation vectors, activation-stationary.
//
// Same arithmetic as the general matvec kernel (per-unit scales applied in
// f32 around an integer-weight inner product), organised for HBM streaming:
//
//  * Each lane owns a fixed set of 32-weight units of a row (u = l, l + LPR,
//    ...), so it loads its slice of x once, precomputes the per-unit sums of
//    x (and, for fp16 W4A16, the fp16 pairs matching the nibble split), and
//    keeps them in registers for every row it visits.
//  * A wave walks row groups with a grid stride.  All weight loads of the
//    next group are issued before the current group is computed (register
//    double buffering), so each wave keeps two groups of 128-bit loads in
//    flight and the first loads leave before anything else happens.
//  * Partial sums are reduced across the LPR lanes of a row with DPP moves
//    inside 16-lane rows and ds_bpermute only across rows.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "qmv_internal.h"

namespace qmv {
namespace {

#ifndef QMV_XS_STAGE16
#define QMV_XS_STAGE16 0  // fp16 activations also staged once per block in LDS
#endif
#ifndef QMV_XS_WAVES
#define QMV_XS_WAVES 4
#endif
constexpr int kWaves = QMV_XS_WAVES;  // waves per block when each wave walks its own row groups
constexpr int kThreads = 64 * kWaves;

typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Weight bytes are read exactly once: load them with the non-temporal hint so
// they stream through the caches without displacing the activations.
#ifndef QMV_NT_WEIGHTS
#define QMV_NT_WEIGHTS 1
#endif
__device__ __forceinline__ uint4 ld_w4(const void* p) {
#if QMV_NT_WEIGHTS
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *static_cast<const uint4*>(p);
#endif
}
__device__ __forceinline__ uint2 ld_w2(const void* p) {
#if QMV_NT_WEIGHTS
  const u32x2 v = __builtin_nontemporal_load(static_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
#else
  return *static_cast<const uint2*>(p);
#endif
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, false));
}

// Sum over each 16-lane row with DPP: afterwards every lane of a row holds the
// row total (rotate by 8, mirror within 8, then swap pairs inside quads).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0x128>(v);  // row_ror:8
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  return v;
}

__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Total of v over the LPR lanes of lane group `sub` (64 / LPR groups per wave).
template <int LPR>
__device__ __forceinline__ float group_sum(float v, int sub) {
  v = row16_sum(v);
  if constexpr (LPR == 64) {
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
  } else if constexpr (LPR == 32) {
    const float a = lane_f(v, 0) + lane_f(v, 16);
    const float b = lane_f(v, 32) + lane_f(v, 48);
    return sub ? b : a;
  } else {
    return v;
  }
}

// gfx950 cross-half swaps, written out: the compiler builtins returned the first
// register for both results in this toolchain.  Each is a register permute
// with both operands read and written; the s_nop pairs give the wait states
// around a VALU write / read of the operands.
__device__ __forceinline__ void swap32(float& a, float& b) {  // a.hi <-> b.lo (32-lane halves)
  asm("s_nop 4\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 4" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16(float& a, float& b) {  // odd 16-lane rows of a <-> even rows of b
  asm("s_nop 4\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 4" : "+v"(a), "+v"(b));
}

// Totals of acc[0 .. R) over all 64 lanes (R rows, each spread over the whole
// wave): afterwards every lane l holds the total of row l / (64 / R).  The
// swaps fold the rows into disjoint lane ranges, so R rows cost 2R - 1
// swaps-and-adds plus one 16-lane DPP sum (R = 4: ~12 instructions, where a
// DPP sum and four readlanes per row took ~44).
template <int R>
__device__ __forceinline__ float wave_rows_sum(const float (&acc)[R]) {
  if constexpr (R == 4) {
    float a0 = acc[0], a1 = acc[1], a2 = acc[2], a3 = acc[3];
    swap32(a0, a2);  // a0 = [row 0 low half, row 2 low half], a2 = [row 0 high half, row 2 high half]
    swap32(a1, a3);
    float s02 = a0 + a2, s13 = a1 + a3;  // 32-lane partials: rows 0 | 2 and 1 | 3
    swap16(s02, s13);
    return row16_sum(s02 + s13);         // 16-lane row j: row j
  } else if constexpr (R == 2) {
    float a0 = acc[0], a1 = acc[1];
    swap32(a0, a1);
    float s = a0 + a1, t = s;            // lanes 0-31: row 0, 32-63: row 1
    swap16(s, t);
    return row16_sum(s + t);
  } else {
    float a = acc[0], b = acc[0];
    swap32(a, b);
    float s = a + b, t = s;
    swap16(s, t);
    return row16_sum(s + t);
  }
}

// ----------------------------------------------------------- per-format units

template <int FMT>
struct Raw;
template <>
struct Raw<QMV_Q8_0> { uint4 q0, q1; uint32_t sc; };
template <>
struct Raw<QMV_W4A16_G64> { uint4 q; uint32_t sz; };
template <>
struct Raw<QMV_Q4K> { uint4 q; uint4 meta; };
template <>
struct Raw<QMV_Q6K> { uint4 q; uint2 qh; uint32_t s2; uint32_t d; };
template <>
struct Raw<QMV_Q4_0> { uint4 q; uint32_t d; };
template <>
struct Raw<QMV_Q5_0> { uint4 q; uint32_t qh; uint32_t d; };
template <>
struct Raw<QMV_Q5K> { uint4 q; uint32_t qh; uint4 meta; };
template <>
struct Raw<QMV_DENSE_BF16> { uint4 q[4]; };
template <>
struct Raw<QMV_I8_ROW> { uint4 q0, q1; uint32_t sc; };

// Weight planes are read through raw buffer resources: an offset at or past
// the plane size returns zeros without touching memory.  Rows past N and row
// groups past the end of a wave's work therefore load unconditionally, so every
// wave issues the same number of loads in the same order and the compiler's
// wait counts stay exact (behind a branch it must assume the fewest loads were
// issued and waits for the newest one).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;  // past every plane (planes are < 2^31 bytes)
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped) 32-bit data, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), kRsrcWord3);
}

// cache policy of the weight-code loads: non-temporal (read once), like ld_w4
constexpr int kNT = QMV_NT_WEIGHTS ? 2 : 0;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
template <int POL>
__device__ __forceinline__ uint4 bl128(rsrc_t r, uint32_t o) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, int(o), 0, POL);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int POL>
__device__ __forceinline__ uint2 bl64(rsrc_t r, uint32_t o) {
  const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, int(o), 0, POL);
  return make_uint2(v.x, v.y);
}

struct Geo {  // buffer resources of the planes
  rsrc_t q, p1, p2, p3;
  int K;
};

// Unit u (32 weights) of `row`; ok = false reads nothing and yields zeros.
template <int FMT>
__device__ __forceinline__ Raw<FMT> load_raw(const Geo& g, int row, int u, bool ok) {
  Raw<FMT> r;
  const uint32_t R = uint32_t(row), K = uint32_t(g.K), U = uint32_t(u);
  const uint32_t bad = ok ? 0u : kOOB;
  if constexpr (FMT == QMV_Q8_0) {
    const uint32_t o = (R * K + 32u * U) | bad;
    r.q0 = bl128<kNT>(g.q, o);
    r.q1 = bl128<kNT>(g.q, o + 16u);
    r.sc = __builtin_amdgcn_raw_buffer_load_b16(g.p1, int(((R * (K >> 5) + U) * 2u) | bad), 0, 0);
  } else if constexpr (FMT == QMV_W4A16_G64) {
    r.q = bl128<kNT>(g.q, (R * (K >> 1) + 16u * U) | bad);
    r.sz = __builtin_amdgcn_raw_buffer_load_b32(g.p1, int(((R * (K >> 6) + (U >> 1)) * 4u) | bad), 0, 0);
  } else if constexpr (FMT == QMV_Q4K) {
    r.q = bl128<kNT>(g.q, (R * (K >> 1) + 16u * U) | bad);
    r.meta = bl128<0>(g.p1, ((R * (K >> 8) + (U >> 3)) * 16u) | bad);
  } else if constexpr (FMT == QMV_Q6K) {
    r.q = bl128<kNT>(g.q, (R * (K >> 1) + 16u * U) | bad);
    r.qh = bl64<kNT>(g.p1, ((R * (K >> 5) + U) * 8u) | bad);
    r.s2 = __builtin_amdgcn_raw_buffer_load_b16(g.p2, int(((R * (K >> 5) + U) * 2u) | bad), 0, 0);
    r.d = __builtin_amdgcn_raw_buffer_load_b16(g.p3, int(((R * (K >> 8) + (U >> 3)) * 2u) | bad), 0, 0);
  } else if constexpr (FMT == QMV_Q4_0) {
    r.q = bl128<kNT>(g.q, (R * (K >> 1) + 16u * U) | bad);
    r.d = __builtin_amdgcn_raw_buffer_load_b16(g.p1, int(((R * (K >> 5) + U) * 2u) | bad), 0, 0);
  } else if constexpr (FMT == QMV_Q5_0) {
    r.q = bl128<kNT>(g.q, (R * (K >> 1) + 16u * U) | bad);
    r.qh = __builtin_amdgcn_raw_buffer_load_b32(g.p1, int(((R * (K >> 5) + U) * 4u) | bad), 0, kNT);
    r.d = __builtin_amdgcn_raw_buffer_load_b16(g.p2, int(((R * (K >> 5) + U) * 2u) | bad), 0, 0);
  } else if constexpr (FMT == QMV_Q5K) {
    r.q = bl128<kNT>(g.q, (R * (K >> 1) + 16u * U) | bad);
    r.qh = __builtin_amdgcn_raw_buffer_load_b32(g.p1, int(((R * (K >> 5) + U) * 4u) | bad), 0, kNT);
    r.meta = bl128<0>(g.p2, ((R * (K >> 8) + (U >> 3)) * 16u) | bad);
  } else if constexpr (FMT == QMV_DENSE_BF16) {
    const uint32_t o = ((R * K + 32u * U) * 2u) | bad;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.q[i] = bl128<kNT>(g.q, o + 16u * i);
  } else {  // QMV_I8_ROW
    const uint32_t o = (R * K + 32u * U) | bad;
    r.q0 = bl128<kNT>(g.q, o);
    r.q1 = bl128<kNT>(g.q, o + 16u);
    r.sc = __builtin_amdgcn_raw_buffer_load_b32(g.p1, int((R * 4u) | bad), 0, 0);
  }
  return r;
}

// Activation slice of one unit, held in registers.
template <bool H2>
struct XUnit;
template <>
struct XUnit<false> { float v[32]; float s0, s1; };   // s0: sum of all 32 (or first 16), s1: last 16
template <>
struct XUnit<true> { half2_t p[16]; float s; };       // fp16 pairs matching the code pairs of unit_dot, sum

// fp16 activations of one unit (32 values, 4 x 16 bytes), fetched from global
// memory before the weight loads are issued.
struct XRaw16 { uint4 v[4]; };
__device__ __forceinline__ XRaw16 fetch_x16(const void* xv, int64_t off) {
  const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + off);
  XRaw16 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = xp[i];
  return r;
}

// fp16 x: from the fetched words `raw`; f32 x: from the block's LDS copy `xv`
// at float offset `off` (a unit's 16-byte words XOR-permuted by the unit
// index, as the staging stores them).  valid = false gives a zero slice.
template <int FMT, bool XF16>
__device__ __forceinline__ void load_x(XUnit<FMT == QMV_W4A16_G64 && XF16>& xu, const void* xv, int64_t off,
                                       bool valid, const XRaw16* raw) {
  if constexpr (FMT == QMV_W4A16_G64 && XF16) {
    float s = 0.0f;
    const half2_t one2 = as_h2(0x3C003C00u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // pairs in the order unit_dot takes the codes of word i: (x0, x2), (x4, x6),
      // (x1, x3), (x5, x7) with x_k = x[8i + k]
      const uint4 xx = valid ? raw->v[i] : make_uint4(0, 0, 0, 0);
      xu.p[4 * i + 0] = as_h2(__builtin_amdgcn_perm(xx.y, xx.x, 0x05040100u));
      xu.p[4 * i + 1] = as_h2(__builtin_amdgcn_perm(xx.w, xx.z, 0x05040100u));
      xu.p[4 * i + 2] = as_h2(__builtin_amdgcn_perm(xx.y, xx.x, 0x07060302u));
      xu.p[4 * i + 3] = as_h2(__builtin_amdgcn_perm(xx.w, xx.z, 0x07060302u));
#pragma unroll
      for (int j = 0; j < 4; ++j) s = __builtin_amdgcn_fdot2(xu.p[4 * i + j], one2, s, false);
    }
    xu.s = s;
  } else if constexpr (XF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 xx = valid ? raw->v[i] : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {xx.x, xx.y, xx.z, xx.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        xu.v[8 * i + 2 * c] = f16_bits_to_f32(w[c] & 0xFFFFu);
        xu.v[8 * i + 2 * c + 1] = f16_bits_to_f32(w[c] >> 16);
      }
    }
  } else {
    const int u = int(off >> 5);
    const float4* xp = reinterpret_cast<const float4*>(static_cast<const float*>(xv) + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float4 xx = valid ? xp[i ^ (u & 7)] : make_float4(0.f, 0.f, 0.f, 0.f);
      xu.v[4 * i] = xx.x; xu.v[4 * i + 1] = xx.y; xu.v[4 * i + 2] = xx.z; xu.v[4 * i + 3] = xx.w;
    }
  }
  if constexpr (!(FMT == QMV_W4A16_G64 && XF16)) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { a += xu.v[i]; b += xu.v[16 + i]; }
    if (FMT == QMV_Q6K) { xu.s0 = a; xu.s1 = b; } else { xu.s0 = a + b; xu.s1 = 0.f; }
  }
}

// acc += contribution of one unit of one row.  `sh` = 6 * (sub-block index within
// the Q4K super-block) for the sc / m fields.
template <int FMT, bool XF16>
__device__ __forceinline__ float unit_dot(const Raw<FMT>& w, const XUnit<FMT == QMV_W4A16_G64 && XF16>& xu,
                                          int sh, float acc) {
  if constexpr (FMT == QMV_W4A16_G64 && XF16) {
    float dot = 0.0f;
    const uint32_t wd[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // word i holds the codes of k = 8i .. 8i + 7, nibble k % 8 at bit 4 (k % 8).
      // Even and odd nibbles become bytes (ev: k = 0, 2, 4, 6; od: 1, 3, 5, 7), and
      // one byte permute puts two of them under 0x64 high bytes: the exact fp16
      // pair (1024 + q_a, 1024 + q_b) for v_dot2 (7 ops per word, was 11)
      const uint32_t ev = wd[i] & 0x0F0F0F0Fu, od = (wd[i] >> 4) & 0x0F0F0F0Fu;
      constexpr uint32_t k64 = 0x64646464u;
      dot = __builtin_amdgcn_fdot2(as_h2(__builtin_amdgcn_perm(k64, ev, 0x04010400u)), xu.p[4 * i + 0], dot, false);
      dot = __builtin_amdgcn_fdot2(as_h2(__builtin_amdgcn_perm(k64, ev, 0x04030402u)), xu.p[4 * i + 1], dot, false);
      dot = __builtin_amdgcn_fdot2(as_h2(__builtin_amdgcn_perm(k64, od, 0x04010400u)), xu.p[4 * i + 2], dot, false);
      dot = __builtin_amdgcn_fdot2(as_h2(__builtin_amdgcn_perm(k64, od, 0x04030402u)), xu.p[4 * i + 3], dot, false);
    }
    const float s = f16_bits_to_f32(w.sz & 0xFFFFu);
    const float zo = 1024.0f + f16_bits_to_f32(w.sz >> 16);  // exact
    return fmaf(s, fmaf(-zo, xu.s, dot), acc);
  } else if constexpr (FMT == QMV_Q8_0 || FMT == QMV_I8_ROW) {
    // codes u = q + 128 as exact fp16 pairs (1024 + u_a, 1024 + u_b), one byte
    // permute per two, each half taken by a mixed-precision FMA against f32 x
    float tx = 0.0f;
    const uint32_t wd[8] = {w.q0.x, w.q0.y, w.q0.z, w.q0.w, w.q1.x, w.q1.y, w.q1.z, w.q1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u = wd[i] ^ 0x80808080u;
      constexpr uint32_t k64 = 0x64646464u;
      const half2_t lo = as_h2(__builtin_amdgcn_perm(k64, u, 0x04010400u));
      const half2_t hi = as_h2(__builtin_amdgcn_perm(k64, u, 0x04030402u));
      tx = fmaf(static_cast<float>(lo[0]), xu.v[4 * i], tx);
      tx = fmaf(static_cast<float>(lo[1]), xu.v[4 * i + 1], tx);
      tx = fmaf(static_cast<float>(hi[0]), xu.v[4 * i + 2], tx);
      tx = fmaf(static_cast<float>(hi[1]), xu.v[4 * i + 3], tx);
    }
    const float ux = fmaf(-1024.0f, xu.s0, tx);  // sum (q + 128) x
    const float sc = FMT == QMV_Q8_0 ? f16_bits_to_f32(w.sc) : __builtin_bit_cast(float, w.sc);
    return fmaf(sc, fmaf(-128.0f, xu.s0, ux), acc);
  } else if constexpr (FMT == QMV_DENSE_BF16) {
    // bf16 pairs: the low half widens by a shift, the high half by a mask
    float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wd[4] = {w.q[i].x, w.q[i].y, w.q[i].z, w.q[i].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        t0 = fmaf(__builtin_bit_cast(float, wd[c] << 16), xu.v[8 * i + 2 * c], t0);
        t1 = fmaf(__builtin_bit_cast(float, wd[c] & 0xFFFF0000u), xu.v[8 * i + 2 * c + 1], t1);
      }
    }
    return acc + (t0 + t1);
  } else {
    // 4- and 6-bit codes b as fp16 pairs (1024 + b_a, 1024 + b_b) (exact: one
    // v_perm_b32 puts two code bytes under 0x64 high bytes), each half taken by
    // a mixed-precision FMA (v_fma_mix_f32) against f32 x: sum b x = sum t x -
    // 1024 sum x
    float ta = 0.0f, tb = 0.0f;
    const uint32_t wd[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t ev = wd[i] & 0x0F0F0F0Fu;         // byte c: q[8i + 2c]
      uint32_t od = (wd[i] >> 4) & 0x0F0F0F0Fu;  // byte c: q[8i + 2c + 1]
      if constexpr (FMT == QMV_Q6K) {
        const uint32_t h = (i >> 1) ? w.qh.y : w.qh.x;
        const int f = (i & 1) * 2;
        ev |= ((h >> (2 * f)) & 0x03030303u) << 4;
        od |= ((h >> (2 * f + 2)) & 0x03030303u) << 4;
      } else if constexpr (FMT == QMV_Q5_0 || FMT == QMV_Q5K) {
        // fifth bits of word i: bit 8c + 2i (+1 for odd) of qh
        ev |= ((w.qh >> (2 * i)) & 0x01010101u) << 4;
        od |= ((w.qh >> (2 * i + 1)) & 0x01010101u) << 4;
      }
      float t = (FMT == QMV_Q6K && i >= 2) ? tb : ta;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        // bytes 2c, 2c + 1 of ev (k = 8i + 4c, + 2) and of od (k = 8i + 4c + 1, + 3)
        constexpr uint32_t k64 = 0x64646464u;
        const uint32_t sel = c ? 0x04030402u : 0x04010400u;
        const half2_t he = as_h2(__builtin_amdgcn_perm(k64, ev, sel));
        const half2_t ho = as_h2(__builtin_amdgcn_perm(k64, od, sel));
        t = fmaf(static_cast<float>(he[0]), xu.v[8 * i + 4 * c], t);
        t = fmaf(static_cast<float>(ho[0]), xu.v[8 * i + 4 * c + 1], t);
        t = fmaf(static_cast<float>(he[1]), xu.v[8 * i + 4 * c + 2], t);
        t = fmaf(static_cast<float>(ho[1]), xu.v[8 * i + 4 * c + 3], t);
      }
      if (FMT == QMV_Q6K && i >= 2) tb = t; else ta = t;
    }
    const float qa = fmaf(-1024.0f, xu.s0, ta);  // sum b x (Q6K: k < 16)
    const float qb = fmaf(-1024.0f, xu.s1, tb);  // Q6K: k >= 16
    if constexpr (FMT == QMV_W4A16_G64) {
      const float s = f16_bits_to_f32(w.sz & 0xFFFFu), z = f16_bits_to_f32(w.sz >> 16);
      return fmaf(s, fmaf(-z, xu.s0, qa), acc);
    } else if constexpr (FMT == QMV_Q4_0 || FMT == QMV_Q5_0) {
      constexpr float off = FMT == QMV_Q4_0 ? 8.0f : 16.0f;
      return fmaf(f16_bits_to_f32(w.d), fmaf(-off, xu.s0, qa), acc);
    } else if constexpr (FMT == QMV_Q4K || FMT == QMV_Q5K) {
      // sc_j sits at bit 6j and m_j at bit 48 + 6j of the 96-bit field {w, z, y};
      // 32-bit funnel shifts read them from any word pair.  (A 64-bit shift
      // wants an aligned register pair, so the compiler copied the loaded words
      // and had to wait for the load right after issuing it.)
      const uint32_t sa = sh < 32 ? w.meta.y : w.meta.z, sb = sh < 32 ? w.meta.z : w.meta.w;
      const uint32_t ma = sh < 16 ? w.meta.z : w.meta.w;
      const float sc = static_cast<float>(__builtin_amdgcn_alignbit(sb, sa, uint32_t(sh) & 31u) & 63u);
      const float m = static_cast<float>(__builtin_amdgcn_alignbit(w.meta.w, ma, uint32_t(sh + 16) & 31u) & 63u);
      const float ds = f16_bits_to_f32(w.meta.x & 0xFFFFu) * sc;
      const float dm = f16_bits_to_f32(w.meta.x >> 16) * m;
      acc = fmaf(ds, qa, acc);
      return fmaf(-dm, xu.s0, acc);
    } else {  // Q6K
      const float d = f16_bits_to_f32(w.d);
      const float s0 = d * static_cast<float>(static_cast<int8_t>(w.s2 & 0xFFu));
      const float s1 = d * static_cast<float>(static_cast<int8_t>(w.s2 >> 8));
      acc = fmaf(s0, fmaf(-32.0f, xu.s0, qa), acc);
      return fmaf(s1, fmaf(-32.0f, xu.s1, qb), acc);
    }
  }
}

// Up to kMaxSeg matrices of one format and one K per launch.  Each segment is
// one matvec (its packed planes, x, y, row count) and owns a contiguous range
// of blocks, sized in proportion to its rows; a block finds its segment once,
// at start, and its waves then stride over that segment's row groups only.
// The table travels in the kernel arguments (no device copy, so launches stay
// graph-capturable).
constexpr int kMaxSeg = 16;
struct Seg {
  const uint8_t* W;
  int64_t off1, off2, off3;
  const void* x;
  float* y;
  int N;
  int b0;   // first block of this segment
  int nb;   // blocks of this segment
  int fmt;  // format (read by the mixed Q4K / Q6K kernel only)
  uint32_t nrec[4];  // bytes of each plane (buffer-resource ranges; each < 2^31)
};
constexpr int kMix = 0;  // FMT of a table mixing Q4K and Q6K segments
// The table is the launch's kernel argument, so its size is paid by every
// launch: kernels take a table of capacity CAP = 1, 4 or 16, the smallest that
// holds the launch's segments (MI355X, grouped 2 x 5632 x 2048 gate+up:
// 5.13 us with a 16-entry table of 1.35 KB, 4.84 us with a 4-entry one).
// Fused epilogue of a single-matrix launch (the pages' decode kernels take the
// biases and the residual adds in their epilogues and run gate / up / SwiGLU
// as one product: aot-llm README, Metal backend notes).  Grouped launches
// leave every pointer null.
struct Epi {
  const uint8_t* W2;   // SwiGLU: the up matrix (same format, shape and planes as the gate)
  const float* bias;   // [N] added to the product, or null
  const float* res;    // [N] residual added last, or null (may be y itself)
};

template <int CAP>
struct SegTableT {
  int first[CAP];  // first block of each segment (INT_MAX past count): one wide scalar load
  Seg s[CAP];
  int count;
  int K;
  Epi ep;
  int pair;        // host only: 1 launches the SwiGLU kernel (one segment, ep.W2 set)
};
using SegTable = SegTableT<kMaxSeg>;  // built on the host, then shrunk to the launch

template <int CAP>
SegTableT<CAP> shrink(const SegTable& t) {  // t.count <= CAP
  SegTableT<CAP> o{};
  for (int i = 0; i < CAP; ++i) {
    o.first[i] = t.first[i];
    o.s[i] = t.s[i];
  }
  o.count = t.count;
  o.K = t.K;
  o.ep = t.ep;
  o.pair = t.pair;
  return o;
}

// FMT / XF16: format and activation type; LPR lanes per row; UPL units per lane
// (covers K = 32 * LPR * UPL * KS, ragged tail masked); R rows per lane group;
// KS: waves that split K between them (1: every wave walks its own row groups
// over the whole of K; KS > 1: the KS waves of a block each take one slice
// of K for the same row groups and their partial sums meet in LDS, added in
// slice order); CAP: table capacity (1: the fields load at fixed offsets,
// with no scan in front of them).
// This block's share of one segment (the body of the kernels below).
// Workgroup barrier for LDS traffic only: __syncthreads() would also wait for
// every weight load in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// y[row] = v when ok; otherwise the store writes nothing (out-of-range offset),
// so every lane issues it and the wait counts stay exact.
__device__ __forceinline__ void store_y(rsrc_t ry, int row, bool ok, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ry, int(ok ? uint32_t(row) * 4u : kOOB), 0, 0);
}

// PAIR: SwiGLU, h = silu(gate row . x) * (up row . x): every row group loads
// the same rows of both matrices (ep.W2 is the up matrix) and the epilogue
// combines the two totals.  Otherwise bias and residual (null: none) are
// added to each total in the epilogue.

// EPI: the bias / residual epilogue (a kernel of its own, so that the plain
// kernels carry none of its registers).
template <int FMT, bool XF16, int LPR, int UPL, int R, int KS, bool DB, bool PAIR = false, bool EPI = false>
__device__ __forceinline__ void xs_segment(const Seg& sg, const int K, const Epi& ep) {
  constexpr int NM = PAIR ? 2 : 1;           // matrices read per row group
  constexpr int TPB = KS == 1 ? kWaves : 1;  // independent lane-group teams per block
  constexpr int BT = 64 * (KS == 1 ? kWaves : KS);  // threads per block
  constexpr bool H2 = (FMT == QMV_W4A16_G64 && XF16);
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int l = lane % LPR;
  const int U = K >> 5;
  const Geo g{make_rsrc(sg.W, sg.nrec[0]), make_rsrc(sg.W + sg.off1, sg.nrec[1]),
              make_rsrc(sg.W + sg.off2, sg.nrec[2]), make_rsrc(sg.W + sg.off3, sg.nrec[3]), K};
  [[maybe_unused]] Geo g2 = g;
  if constexpr (PAIR)
    g2 = Geo{make_rsrc(ep.W2, sg.nrec[0]), make_rsrc(ep.W2 + sg.off1, sg.nrec[1]),
             make_rsrc(ep.W2 + sg.off2, sg.nrec[2]), make_rsrc(ep.W2 + sg.off3, sg.nrec[3]), K};
  const int N = sg.N;
  // the value stored from a row's total(s); eb / er: its bias and residual,
  // loaded with the row group's weights (load_epi) so that their latency is
  // not added at the end
  auto finish = [&](float tot, float tot2, float eb, float er) -> float {
    if constexpr (PAIR) {
      return silu_mul(tot, tot2);
    } else if constexpr (EPI) {
      float v = tot;
      if (ep.bias) v += eb;
      if (ep.res) v = er + v;
      return v;
    } else {
      return tot;
    }
  };
  const rsrc_t ry = make_rsrc(sg.y, uint32_t(N) * 4u);
  const int ngroups = (N + R * RPW - 1) / (R * RPW);
  // wave-uniform (readfirstlane): the loop's branches and loads stay scalar-controlled
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = (int(blockIdx.x) - sg.b0) * TPB + (KS == 1 ? wv : 0);
  const int TW = sg.nb * TPB;
  const int ks = KS == 1 ? 0 : wv;  // K slice of this wave
  __shared__ float red[2][KS][NM * RPW * R];
  int par = 0;

  int uu[UPL], sh[UPL];
  bool uv[UPL];
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int u = (ks * UPL + j) * LPR + l;
    uv[j] = u < U;
    uu[j] = uv[j] ? u : U - 1;
    sh[j] = 6 * (uu[j] & 7);
  }

  // 1. activations first.  With f32 x (and fp16 x when STAGE16) the block
  // copies the whole vector into LDS: every wave of the block reads the same
  // vector, so this keeps the per-lane activation loads (128 bytes per unit
  // for f32) off the vector-memory path.  Otherwise each lane fetches its own
  // fp16 slice.
  constexpr bool STAGE = !XF16 || QMV_XS_STAGE16;
  constexpr int XF = 32 * LPR * UPL * KS;          // activations this configuration covers
  constexpr int XW = XF16 ? XF / 8 : XF / 4;       // ... in 16-byte words
  constexpr int NXI = (XW + BT - 1) / BT;          // staging loads per thread
  // staged words in one vector value (a private array here was placed in LDS
  // by the compiler, which waited for each load before the weights went out)
  typedef uint32_t xstage_t __attribute__((ext_vector_type(STAGE ? 4 * NXI : 4)));
  [[maybe_unused]] xstage_t xst;
  [[maybe_unused]] XRaw16 xr[XF16 ? UPL : 1];
  if constexpr (STAGE) {
    const uint4* xg = static_cast<const uint4*>(sg.x);
    const int nw = XF16 ? (K >> 3) : (K >> 2);
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
      const uint4 t = xg[min(int(threadIdx.x) + i * BT, nw - 1)];
      xst[4 * i] = t.x; xst[4 * i + 1] = t.y; xst[4 * i + 2] = t.z; xst[4 * i + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < UPL; ++j) xr[j] = fetch_x16(sg.x, 32 * uu[j]);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight loads

  // 2. weights of this wave's first two row groups (one with DB = false):
  // both register sets in flight before anything waits (groups past the end
  // read nothing)
  Raw<FMT> ga[NM][R][UPL], gb[NM][R][UPL];  // two register sets, used in turn (no copies)
  auto load_group = [&](Raw<FMT> (&dst)[NM][R][UPL], int gi) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = gi * (R * RPW) + r * RPW + sub;
#pragma unroll
        for (int j = 0; j < UPL; ++j) dst[m][r][j] = load_raw<FMT>(m ? g2 : g, row, uu[j], row < N && uv[j]);
      }
  };
  // bias / residual of a row group's rows (row r * RPW + sub of the group;
  // rows past the end clamped), issued after its weights
  float eba[R], era[R], ebb[R], erb[R];
  auto load_epi = [&](float (&eb)[R], float (&er)[R], int gi) {
    if constexpr (EPI) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int rc = min(gi * (R * RPW) + r * RPW + sub, N - 1);
        eb[r] = ep.bias ? ep.bias[rc] : 0.0f;
        er[r] = ep.res ? ep.res[rc] : 0.0f;
      }
    }
  };
  int grp = gw;
  load_group(ga, grp);
  if constexpr (DB) load_group(gb, grp + TW);
  load_epi(eba, era, grp);
  if constexpr (DB) load_epi(ebb, erb, grp + TW);

  // 3. activation slices into registers (and the per-unit sums)
  XUnit<H2> xs[UPL];
  if constexpr (STAGE) {
    __shared__ uint4 xl[NXI * BT];  // XW rounded up to whole staging rounds
    // 16-byte word w at w ^ ((w / 8) % 8) (within its 128-byte row): the lanes
    // of a row, which read the same word of different units at once, hit
    // different banks (f32: word c of unit u at 8u + (c ^ (u % 8)); linear, the
    // 16 lanes 128 bytes apart all fell on the same 4 banks)
#pragma unroll
    for (int i = 0; i < NXI; ++i) {  // unconditional: no load sinks into a branch
      const int w = int(threadIdx.x) + i * BT;
      xl[w ^ ((w >> 3) & 7)] = make_uint4(xst[4 * i], xst[4 * i + 1], xst[4 * i + 2], xst[4 * i + 3]);
    }
    lds_barrier();
    if constexpr (XF16) {
#pragma unroll
      for (int j = 0; j < UPL; ++j) {
        XRaw16 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int wi = 4 * uu[j] + i;  // fp16: 4 words per unit
          w.v[i] = xl[wi ^ ((wi >> 3) & 7)];
        }
        load_x<FMT, XF16>(xs[j], nullptr, 0, uv[j], &w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < UPL; ++j) load_x<FMT, XF16>(xs[j], xl, 32 * uu[j], uv[j], nullptr);
    }
  } else {
#pragma unroll
    for (int j = 0; j < UPL; ++j) load_x<FMT, XF16>(xs[j], nullptr, 0, uv[j], &xr[j]);
  }

  auto do_group = [&](const Raw<FMT> (&cur)[NM][R][UPL], int gi, const float (&eb)[R], const float (&er)[R]) {
    float acc[NM][R];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      if (uv[j]) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int r = 0; r < R; ++r) acc[m][r] = unit_dot<FMT, XF16>(cur[m][r][j], xs[j], sh[j], acc[m][r]);
      }
    }
    if constexpr (LPR == 64 && (R == 1 || R == 2 || R == 4)) {
      // one row per lane range: lane l holds row r = l / (64 / R)
      const float tot = wave_rows_sum<R>(acc[0]);
      const float tot2 = PAIR ? wave_rows_sum<R>(acc[NM - 1]) : 0.0f;
      const int r = lane / (64 / R);
      const bool first = lane % (64 / R) == 0;
      const int row = gi * R + r;
      if constexpr (KS == 1) {
        float b = eb[0], e = er[0];  // this lane's row r (a select, not a dynamic register index)
#pragma unroll
        for (int i = 1; i < R; ++i) {
          b = r == i ? eb[i] : b;
          e = r == i ? er[i] : e;
        }
        store_y(ry, row, first && row < N, finish(tot, tot2, b, e));
      } else {
        if (first) {
          red[par][ks][r] = tot;
          if constexpr (PAIR) red[par][ks][RPW * R + r] = tot2;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float tot = group_sum<LPR>(acc[0][r], sub);
        const float tot2 = PAIR ? group_sum<LPR>(acc[NM - 1][r], sub) : 0.0f;
        const int row = gi * (R * RPW) + r * RPW + sub;
        if constexpr (KS == 1) {
          store_y(ry, row, l == 0 && row < N, finish(tot, tot2, eb[r], er[r]));
        } else {
          if (l == 0) {
            red[par][ks][r * RPW + sub] = tot;
            if constexpr (PAIR) red[par][ks][RPW * R + r * RPW + sub] = tot2;
          }
        }
      }
    }
    if constexpr (KS > 1) {  // every wave of the block runs the same groups: uniform barrier
      lds_barrier();
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = gi * (R * RPW) + r * RPW + sub;
        float t = 0.0f, t2 = 0.0f;
#pragma unroll
        for (int w = 0; w < KS; ++w) {
          t += red[par][w][r * RPW + sub];
          if constexpr (PAIR) t2 += red[par][w][RPW * R + r * RPW + sub];
        }
        store_y(ry, row, ks == 0 && l == 0 && row < N, finish(t, t2, eb[r], er[r]));
      }
      par ^= 1;  // the next group writes the other buffer while this one is read
    }
  };
  if constexpr (DB) {
    // a set is refilled as soon as it has been used, so the other set's loads
    // are always in flight while one group is computed
    while (grp < ngroups) {
      do_group(ga, grp, eba, era);
      load_group(ga, grp + 2 * TW);
      load_epi(eba, era, grp + 2 * TW);
      if (grp + TW >= ngroups) break;
      do_group(gb, grp + TW, ebb, erb);
      load_group(gb, grp + 3 * TW);
      load_epi(ebb, erb, grp + 3 * TW);
      grp += 2 * TW;
    }
  } else {  // at most one group per wave (the launcher checks)
    if (grp < ngroups) do_group(ga, grp, eba, era);
  }
}

// DB: each wave may take several row groups (two register sets in turn);
// false when every wave has at most one.
template <int FMT, bool XF16, int LPR, int UPL, int R, int CAP, int KS, bool DB>
__global__ __launch_bounds__(KS == 1 ? kThreads : 64 * KS) void matvec_xs_kernel(const SegTableT<CAP> t) {
  // this block's segment (block-uniform scan of at most CAP entries)
  // (unused table entries start at INT_MAX, so this is a count over all
  // entries, read with one wide scalar load, where a loop to t.count waited
  // for each entry in turn before the first weight load went out)
  int si = 0;
  if constexpr (CAP > 1) {
#pragma unroll
    for (int i = 1; i < CAP; ++i) si += int(blockIdx.x) >= t.first[i] ? 1 : 0;
  }
  xs_segment<FMT, XF16, LPR, UPL, R, KS, DB>(t.s[si], t.K, t.ep);
}

// One matvec with the bias / residual epilogue (t.ep).
template <int FMT, bool XF16, int LPR, int UPL, int R, int KS, bool DB>
__global__ __launch_bounds__(KS == 1 ? kThreads : 64 * KS) void matvec_xs_epi_kernel(const SegTableT<1> t) {
  xs_segment<FMT, XF16, LPR, UPL, R, KS, DB, false, true>(t.s[0], t.K, t.ep);
}

// SwiGLU of one gate / up pair: one segment (the gate), ep.W2 the up matrix.
template <int FMT, bool XF16, int LPR, int UPL, int R, int KS, bool DB>
__global__ __launch_bounds__(KS == 1 ? kThreads : 64 * KS) void matvec_xs_pair_kernel(const SegTableT<1> t) {
  xs_segment<FMT, XF16, LPR, UPL, R, KS, DB, true>(t.s[0], t.K, t.ep);
}

// Q4K and Q6K segments in one launch (the K-quant mix of one decoder layer's
// q / k / v projections): each block takes its own segment's format path.
template <int LPR, int UPL, int R, int KS, bool DB, int CAP>
__global__ __launch_bounds__(KS == 1 ? kThreads : 64 * KS) void matvec_xs_mix_kernel(const SegTableT<CAP> t) {
  int si = 0;
#pragma unroll
  for (int i = 1; i < CAP; ++i) si += int(blockIdx.x) >= t.first[i] ? 1 : 0;
  const Seg& sg = t.s[si];
  if (sg.fmt == QMV_Q6K) xs_segment<QMV_Q6K, false, LPR, UPL, R, KS, DB>(sg, t.K, t.ep);
  else xs_segment<QMV_Q4K, false, LPR, UPL, R, KS, DB>(sg, t.K, t.ep);
}

bool double_buffer_forced() {
  static const bool v = [] {
    return ab_switch("QMV_MATVEC_DB", 0) == 1;  // A/B tuning only: 1 keeps both register sets always
  }();
  return v;
}

template <int FMT, bool XF16, int LPR, int UPL, int R, int KS>
hipError_t go(SegTable& t, hipStream_t s) {
  constexpr int BW = KS == 1 ? kWaves : KS;   // waves per block
  constexpr int TPB = KS == 1 ? kWaves : 1;   // row-group teams per block
  constexpr int rows_per_group = R * (64 / LPR);
  int64_t groups[kMaxSeg], total = 0;
  for (int i = 0; i < t.count; ++i) {
    groups[i] = (t.s[i].N + rows_per_group - 1) / rows_per_group;
    total += groups[i];
  }
  // Waves per CU the grid may fill: 16, or, with fp16 activations, up to 24
  // when that gives every row group a wave of its own (measured: grouped
  // 2 x 5632 x 2048 W4A16, 5632 groups, 2 % faster than at 16, where some waves
  // take two groups; the f32-activation paths and the large heads ran slower
  // with more waves).
  constexpr bool H2 = (FMT == QMV_W4A16_G64 && XF16);
  static const int waves_forced = [] {  // A/B tuning only: waves per CU the grid may fill
    const int v = ab_switch("QMV_MATVEC_WAVES_CU", 0);
    return (v >= 4 && v <= 32) ? v : 0;
  }();
  const int64_t max_blocks =
      256 * (waves_forced ? waves_forced : (H2 && total * KS <= 256 * 24) ? 24 : 16) / BW;
  const int64_t budget = std::min<int64_t>((total + TPB - 1) / TPB, max_blocks);
  int b = 0;
  for (int i = 0; i < t.count; ++i) {
    const int64_t need = (groups[i] + TPB - 1) / TPB;
    const int64_t share = (budget * groups[i] + total - 1) / total;
    t.s[i].b0 = b;
    t.s[i].nb = int(std::max<int64_t>(1, std::min(need, share)));
    b += t.s[i].nb;
  }
  for (int i = 0; i < kMaxSeg; ++i) t.first[i] = i < t.count ? t.s[i].b0 : INT_MAX;  // INT_MAX: never selected
  // one row group per team everywhere: no second register set (its loads would
  // all fall past the end)
  bool single = !double_buffer_forced();
  for (int i = 0; i < t.count; ++i) single = single && groups[i] <= int64_t(t.s[i].nb) * TPB;
  const dim3 grid(b), block(64 * BW);
  auto launch = [&](auto db) {
    constexpr bool DB = decltype(db)::value;
    if constexpr (FMT == kMix) {  // a mix has two segments at least
      if (t.count <= 4)
        hipLaunchKernelGGL((matvec_xs_mix_kernel<LPR, UPL, R, KS, DB, 4>), grid, block, 0, s, shrink<4>(t));
      else
        hipLaunchKernelGGL((matvec_xs_mix_kernel<LPR, UPL, R, KS, DB, kMaxSeg>), grid, block, 0, s, t);
    } else {
      if (t.pair) {
        // two matrices' registers per row group: at most two rows x units per lane
        if constexpr (R * UPL <= 2)
          hipLaunchKernelGGL((matvec_xs_pair_kernel<FMT, XF16, LPR, UPL, R, KS, DB>), grid, block, 0, s, shrink<1>(t));
      } else if (t.ep.bias || t.ep.res) {  // a single matrix
        hipLaunchKernelGGL((matvec_xs_epi_kernel<FMT, XF16, LPR, UPL, R, KS, DB>), grid, block, 0, s, shrink<1>(t));
      } else if (t.count == 1)
        hipLaunchKernelGGL((matvec_xs_kernel<FMT, XF16, LPR, UPL, R, 1, KS, DB>), grid, block, 0, s, shrink<1>(t));
      else if (t.count <= 4)
        hipLaunchKernelGGL((matvec_xs_kernel<FMT, XF16, LPR, UPL, R, 4, KS, DB>), grid, block, 0, s, shrink<4>(t));
      else
        hipLaunchKernelGGL((matvec_xs_kernel<FMT, XF16, LPR, UPL, R, kMaxSeg, KS, DB>), grid, block, 0, s, t);
    }
  };
  if (single) launch(std::false_type{});
  else launch(std::true_type{});
  return hipGetLastError();
}

// Rows per lane group R.  One row when the launch has at most 1024 row slots
// (rows / rows read side by side per wave): the launch is latency-bound and
// waves count.  Otherwise two, or four with fp16 W4A16 activations and K in
// one wave, measured on MI355X with the static load schedule (grouped
// 2 x 5632 x 2048 W4A16 gate+up: R = 1 / 2 / 4: 5.82 / 5.89 / 5.48 us; the
// K-split 2048 x 5632 down: 4.38 / 4.10 / 4.36 us; the 32000 x 2048 Q6K head
// and the 151936 x 1024 Q4K head are best at two).  R = 8 (fp16 W4A16, K in
// one wave) only through the tuning switch.
template <int FMT, bool XF16, int LPR, int UPL, int KS = 1>
hipError_t pick_r(SegTable& t, int rsel, hipStream_t s) {
  constexpr bool H2 = (FMT == QMV_W4A16_G64 && XF16);
  int64_t rows = 0;
  for (int i = 0; i < t.count; ++i) rows += t.s[i].N;
  const int64_t slots = rows / (64 / LPR);
  // f32 x with K in one wave: four rows when that, and not two, gives every
  // wave a single row group (16 waves per CU; grouped 2 x 5632 x 2048 Q4K
  // gate+up 6.27 -> 5.65 us, where smaller launches and the large heads were
  // slower at four)
  const bool four_fits = KS == 1 && LPR == 64 && rows / 2 > 256 * 16 && (rows + 3) / 4 <= 256 * 16;
  int r = rsel ? rsel : slots <= 1024 ? 1 : ((H2 && KS == 1) || four_fits) ? 4 : 2;
  if constexpr (FMT == QMV_DENSE_BF16) r = r > 2 ? 2 : r;  // 16 weight registers per unit and row
  if (t.pair) r = UPL >= 2 ? 1 : (r > 2 ? 2 : r);          // SwiGLU: two matrices' registers
  if constexpr (H2 && KS == 1 && UPL == 1) {
    if (r == 8) return go<FMT, XF16, LPR, UPL, 8, KS>(t, s);
  } else {
    r = r == 8 ? 4 : r;
  }
  if constexpr (FMT != QMV_DENSE_BF16) {
    if (r == 4) return go<FMT, XF16, LPR, UPL, 4, KS>(t, s);
  }
  return r == 2 ? go<FMT, XF16, LPR, UPL, 2, KS>(t, s) : go<FMT, XF16, LPR, UPL, 1, KS>(t, s);
}

bool ksplit_off() {
  static const bool v = [] {
    return ab_switch("QMV_MATVEC_KSPLIT", 1) == 0;  // A/B tuning only: 0 keeps K in one wave
  }();
  return v;
}

template <int FMT, bool XF16>
bool dispatch(SegTable& t, int rsel, hipStream_t s, hipError_t* e) {
  constexpr bool H2 = (FMT == QMV_W4A16_G64 && XF16);
  const int U = t.K / 32;
  static const int lpr_forced = [] {  // A/B tuning only: lanes per row (16, 32 or 64)
    const int v = ab_switch("QMV_MATVEC_LPR", 0);
    return (v == 16 || v == 32 || v == 64) ? v : 0;
  }();
  int lpr = U >= 64 ? 64 : (U > 16 ? 32 : 16);
  // 17..32 units on a streaming launch (more 4-row groups than the grid holds
  // waves, so every wave walks several groups): 16 lanes per row with two
  // units each and one row per lane group (measured on MI355X, 151936 x 1024
  // Q4K head: 20.2 -> 18.6 us; the 3072 x 1024 up projection, one group per
  // wave, was slower: 3.08 -> 3.29 us)
  int64_t rows = 0;
  for (int i = 0; i < t.count; ++i) rows += t.s[i].N;
  if (lpr == 32 && U <= 32 && rows > 4 * 256 * 16) {
    lpr = 16;
    if (!rsel) rsel = 1;
  }
  if (lpr_forced && lpr_forced < lpr && (U + lpr_forced - 1) / lpr_forced <= 2) lpr = lpr_forced;
  const int upl = (U + lpr - 1) / lpr;
  // activation registers per unit: 17 (fp16 pairs) or 34 (f32)
  if (upl > (H2 ? 4 : 3)) return false;
  // Wide K (more than one unit per lane): split K over upl waves of one unit
  // each instead (measured on MI355X, 2048 x 5632 down projections: W4A16
  // 4.64 -> 4.24 us, Q6K 7.46 -> 7.15 us): less work and fewer activation
  // registers per wave, and a wave's partial sum is ready sooner.
  if (lpr == 64 && upl >= 2 && !ksplit_off()) {
    switch (upl) {
      case 2: *e = pick_r<FMT, XF16, 64, 1, 2>(t, rsel, s); return true;
      case 3: *e = pick_r<FMT, XF16, 64, 1, 3>(t, rsel, s); return true;
      default: *e = pick_r<FMT, XF16, 64, 1, 4>(t, rsel, s); return true;
    }
  }
  if (lpr == 64) {
    switch (upl) {
      case 1: *e = pick_r<FMT, XF16, 64, 1>(t, rsel, s); return true;
      case 2: *e = pick_r<FMT, XF16, 64, 2>(t, rsel, s); return true;
      case 3: *e = pick_r<FMT, XF16, 64, 3>(t, rsel, s); return true;
      default:
        if constexpr (H2) { *e = pick_r<FMT, XF16, 64, 4>(t, rsel, s); return true; }
        return false;
    }
  }
  if (lpr == 32) {
    *e = upl == 1 ? pick_r<FMT, XF16, 32, 1>(t, rsel, s) : pick_r<FMT, XF16, 32, 2>(t, rsel, s);
    return true;
  }
  *e = upl == 1 ? pick_r<FMT, XF16, 16, 1>(t, rsel, s) : pick_r<FMT, XF16, 16, 2>(t, rsel, s);
  return true;
}

int rows_override() {
  static const int v = [] {
    const int r = ab_switch("QMV_MATVEC_ROWS", 0);  // A/B tuning only: rows per lane group (1, 2, 4 or 8)
    return (r == 1 || r == 2 || r == 4 || r == 8) ? r : 0;
  }();
  return v;
}

bool launch_table(int fmt, SegTable& t, int x_dtype, hipStream_t s, hipError_t* err) {
  if (x_dtype == QMV_Q8X) return false;  // 8-bit activations run on the general kernel
  const int rsel = rows_override();
  const bool f16 = (x_dtype == QMV_F16);
  switch (fmt) {
    case QMV_Q8_0: return dispatch<QMV_Q8_0, false>(t, rsel, s, err);
    case QMV_W4A16_G64:
      return f16 ? dispatch<QMV_W4A16_G64, true>(t, rsel, s, err) : dispatch<QMV_W4A16_G64, false>(t, rsel, s, err);
    case QMV_Q4K: return dispatch<QMV_Q4K, false>(t, rsel, s, err);
    case QMV_Q6K: return dispatch<QMV_Q6K, false>(t, rsel, s, err);
    case QMV_Q4_0: return dispatch<QMV_Q4_0, false>(t, rsel, s, err);
    case QMV_Q5_0: return dispatch<QMV_Q5_0, false>(t, rsel, s, err);
    case QMV_Q5K: return dispatch<QMV_Q5K, false>(t, rsel, s, err);
    case QMV_DENSE_BF16: return dispatch<QMV_DENSE_BF16, false>(t, rsel, s, err);
    case QMV_I8_ROW: return dispatch<QMV_I8_ROW, false>(t, rsel, s, err);
    case kMix: return dispatch<kMix, false>(t, rsel, s, err);
    default: return false;
  }
}

// The kernels address each plane with 32-bit buffer offsets and use offsets
// from 2^31 up as "read nothing": every plane must stay below 2^31 bytes.
bool planes_fit(const Planes& p) {
  for (int i = 0; i < p.count; ++i)
    if (p.bytes[i] >= (int64_t(1) << 31)) return false;
  return true;
}

Seg make_seg(int fmt, int64_t N, int64_t K, const void* W, const void* x, void* y) {
  const Planes p = planes_of(fmt, N, K);
  Seg sg{static_cast<const uint8_t*>(W), p.off[1], p.off[2], p.off[3], x, static_cast<float*>(y), int(N), 0, 0, fmt,
         {0, 0, 0, 0}};
  for (int i = 0; i < p.count; ++i) sg.nrec[i] = uint32_t(p.bytes[i]);
  return sg;
}

}  // namespace

// Single-vector matvec on the activation-stationary kernels.  Returns false
// (nothing launched) when the shape needs more activation registers than
// these kernels hold, or has a plane of 2^31 bytes or more; the caller then
// uses the general kernel.
bool launch_matvec_b1(int fmt, int64_t N, int64_t K, const uint8_t* W, const void* x, int x_dtype,
                      float* y, hipStream_t s, hipError_t* err) {
  return launch_matvec_b1_epi(fmt, N, K, W, nullptr, x, x_dtype, y, nullptr, nullptr, s, err);
}

// The same with a fused epilogue: W2 != null runs SwiGLU (y = silu(W x) * (W2 x)),
// otherwise bias / res (null: none) are added to the products.
bool launch_matvec_b1_epi(int fmt, int64_t N, int64_t K, const uint8_t* W, const uint8_t* W2, const void* x,
                          int x_dtype, float* y, const float* bias, const float* res, hipStream_t s,
                          hipError_t* err) {
  if (!planes_fit(planes_of(fmt, N, K))) return false;
  SegTable t{};
  t.count = 1;
  t.K = int(K);
  t.s[0] = make_seg(fmt, N, K, W, x, y);
  t.ep = Epi{W2, bias, res};
  t.pair = W2 != nullptr;
  return launch_table(fmt, t, x_dtype, s, err);
}

// Several single-vector matvecs of one K in one launch per kMaxSeg items.
// Items of one format share a launch; items that are exactly Q4K and Q6K share
// the mixed kernel; any other mix runs one launch series per format.  An item's
// format is its own fmt field, or `fmt` where that is 0.  Returns false
// (nothing launched) when the shape does not fit the activation-stationary
// kernels.
bool launch_matvec_grouped_b1(int fmt, int64_t K, int count, const qmv_matvec_item* items, int x_dtype,
                              hipStream_t s, hipError_t* err) {
  if (x_dtype == QMV_Q8X) return false;  // 8-bit activations run on the general kernel
  const int U = int(K) / 32;
  const int lpr = U >= 64 ? 64 : (U > 16 ? 32 : 16);
  const int upl = (U + lpr - 1) / lpr;
  if (upl > (x_dtype == QMV_F16 ? 4 : 3)) return false;
  auto eff = [&](int i) { return items[i].fmt ? items[i].fmt : fmt; };
  for (int i = 0; i < count; ++i)  // decided before anything is launched
    if (!planes_fit(planes_of(eff(i), items[i].N, K))) return false;
  // launches over the items with indices idx[0..n), as tables of format tfmt
  auto run = [&](int tfmt, const int* idx, int n) {
    const int64_t max_rows = int64_t(1) << 30;  // a launch takes up to kMaxSeg items and 2^30 rows
    for (int i0 = 0; i0 < n;) {
      SegTable t{};
      t.K = int(K);
      int64_t rows = 0;
      while (t.count < kMaxSeg && i0 + t.count < n && (t.count == 0 || rows + items[idx[i0 + t.count]].N <= max_rows)) {
        const int i = idx[i0 + t.count];
        const qmv_matvec_item& it = items[i];
        t.s[t.count++] = make_seg(eff(i), it.N, K, it.W, it.x, it.y);
        rows += it.N;
      }
      if (!launch_table(tfmt, t, x_dtype, s, err)) return false;
      if (*err != hipSuccess) return true;
      i0 += t.count;
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
    return run(same ? eff(0) : kMix, idx, count);
  }
  for (int f = 1; f <= kNumFormats; ++f) {  // one launch series per format present
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
