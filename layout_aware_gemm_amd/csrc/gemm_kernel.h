// Matrix-core (MFMA) bf16 GEMM for gfx950 with layout flags and fused
// epilogues.  Included by one translation unit per operand layout.
//
// Structure of one workgroup (256 threads = 4 wave64s in a 2x2 grid):
//   * it owns a BM x BN output tile and walks K in steps of 64;
//   * operand panels reach LDS one of two ways.  Interior tiles with both
//     operands K-contiguous (NT) copy them straight from global memory into
//     LDS (buffer loads with an LDS destination; three B panels and two A
//     panels for 256x256 tiles, a ring of k32 stages for 128x128).  Every
//     other case -- an operand contiguous along M or N, the fp8 cast, edge
//     tiles -- loads 16-byte vectors along the operand's contiguous axis
//     into registers a k-step ahead and then writes them to the other half
//     of a double-buffered LDS tile;
//   * LDS always holds both panels K-contiguous ([rows][64] bf16, 128 B per
//     row) with the 16-byte chunks XOR-swizzled, so the matrix-core operand
//     reads below are identical for every layout.  An operand that is
//     contiguous along M or N (A 'T', B 'N') is transposed in registers
//     (8x8 / 4x8 blocks of bf16) on its way into LDS;
//   * each wave multiplies its (BM/2) x (BN/2) sub-tile with
//     v_mfma_f32_32x32x16_bf16, fp32 accumulation in registers.
//
// Because the LDS image and the instruction stream after it do not depend
// on the layout, the four layouts produce bitwise-identical results.
#pragma once

#include <type_traits>

#include "bf16_cvt.h"
#include "ce_grad.h"
#include "tgemm_internal.h"

#ifndef TGEMM_MIX
#define TGEMM_MIX 1
#endif

namespace tgemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBK = 64;          // k elements per LDS row
constexpr float kLog2e = 1.4426950408889634f;

// Physical 16-byte chunk of logical chunk c in LDS row `row` (128 B) is
// c ^ ((row >> 1) & 7).  The LDS serves a 16-byte-per-lane access 16 lanes
// at a time across 64 banks (256 B); an LDS row covers half of them, so two
// rows of equal parity compete for the same half.  With this XOR, the 16
// consecutive rows read by 16 lanes (same logical chunk) land in 16
// distinct 16-byte bank groups.  The DMA writer stores 1 KB contiguously
// per instruction and the K-contiguous loader writes two whole rows per 16
// lanes, so both are conflict-free too.  The XOR depends on the row only
// through (row >> 1) & 7, so a lane's fragment addresses in successive
// 32-row blocks differ by immediate offsets.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ uint32_t u4comp(const uint4& v, int d) {
  return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// ----------------------------------------------------------------------
// fp8 (e4m3fn) operands made on load ("Improve the Inductor generated
// kernel for the pattern of output1 = pointwise(input); output2 =
// transpose(output1)", the example: scale, clamp to the largest finite
// e4m3fn value, cast).  Two bf16 values: fp32(x) * s (one rounding), clamp
// to [-448, 448] with NaN kept, then v_cvt_pk_fp8_f32, whose rounding on
// gfx950 is the OCP e4m3fn one (nearest, ties to even; it turns a
// magnitude that rounds past 448 into NaN, hence the clamp, and its scaled
// form only scales by powers of two).  The e4m3fn values go back to bf16,
// which holds each of them exactly, so the bf16 matrix cores multiply the
// fp8 operands exactly.
// ----------------------------------------------------------------------
constexpr float kE4m3Max = 448.0f;

typedef float f32x2_t __attribute__((ext_vector_type(2)));

#if defined(__HIP_DEVICE_COMPILE__)
// fp32(bf16) * s, clamped to [-448, 448] by the IEEE 754-2019 minimum and
// maximum (v_minimum3 / v_maximum3), which keep a NaN a NaN
__device__ __forceinline__ float q8_scaled(uint32_t bf16_in_high_half, float s) {
  const float y = __fmul_rn(__uint_as_float(bf16_in_high_half), s);
  return __builtin_elementwise_minimum(__builtin_elementwise_maximum(y, -kE4m3Max), kE4m3Max);
}

// the high halves of two fp32 values (exact: an e4m3fn value has at most 4
// significant bits) as a bf16 pair
__device__ __forceinline__ uint32_t hi_halves(f32x2_t f) {
  return __builtin_amdgcn_perm(__float_as_uint(f.y), __float_as_uint(f.x), 0x07060302u);
}
#endif

// The e4m3fn codes of the 8 bf16 values of one 16-byte vector: two packed
// conversions fill one register with four codes (x: elements 0-3, y: 4-7,
// element e in byte e % 4).
__device__ __forceinline__ uint2 q8_codes(const uint4& v, float s) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  int c[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = w[2 * h], b = w[2 * h + 1];
    // (the first conversion's other half is overwritten by the second)
    const int t = __builtin_amdgcn_cvt_pk_fp8_f32(q8_scaled(a << 16, s),
                                                  q8_scaled(a & 0xffff0000u, s), (int)a, false);
    c[h] = __builtin_amdgcn_cvt_pk_fp8_f32(q8_scaled(b << 16, s), q8_scaled(b & 0xffff0000u, s),
                                           t, true);
  }
  return make_uint2((uint32_t)c[0], (uint32_t)c[1]);
#else
  (void)v, (void)s;
  return make_uint2(0, 0);
#endif
}

// Cast the 8 bf16 values of one loaded 16-byte vector in place: the codes
// of q8_codes, each register converted back as two pairs.
__device__ __forceinline__ void q8_vec(uint4& v, float s) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint2 c = q8_codes(v, s);
  v.x = hi_halves(__builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false));
  v.y = hi_halves(__builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true));
  v.z = hi_halves(__builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false));
  v.w = hi_halves(__builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true));
#else
  (void)v, (void)s;
#endif
}

// ----------------------------------------------------------------------
// Cross-entropy gradient operand made on load: the 8 bf16 values of one
// loaded vector are 8 consecutive vocabulary columns n0 .. n0+7 of token t
// of the stored e = bf16(exp(y - m_b)); each becomes bf16(e * s - [label])
// with s the scale of the token's 64-column chunk (ce_grad_value, the
// arithmetic of the rescale pass, so the bits are the same).  Elements
// outside the gradient (zero-filled edges) stay zero.
// ----------------------------------------------------------------------
// The scale of token t's chunk and the label's offset from n0 (-1: no
// label column in this vector); zero-filled elements get scale 0.
__device__ __forceinline__ void g_params(const GemmParams& p, int t, int n0, float& s, int& rel) {
  s = 0.f;
  rel = -1;
  if (t < p.gtok && n0 < p.gvoc) {
    s = p.gscale[(int64_t)(n0 / kCeScaleCols) * p.gtok + t];
    rel = p.glabels[t] - n0;
  }
}

__device__ __forceinline__ void g_vec(uint4& v, float s, int rel) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = pack_bf16x2(ce_grad_value(w[q] & 0xffffu, s, rel == 2 * q),
                       ce_grad_value(w[q] >> 16, s, rel == 2 * q + 1));
  v = make_uint4(w[0], w[1], w[2], w[3]);
}

// One dword (two elements) of a gradient vector without the label column:
// each element only multiplied, with g_vec's bits (ce_grad_value without
// the label is fma(e, s, 0)).
__device__ __forceinline__ uint32_t g_dword_scale(uint32_t w, float s) {
  return pack_bf16x2(__fmaf_rn(__uint_as_float(w << 16), s, 0.f),
                     __fmaf_rn(__uint_as_float(w & 0xffff0000u), s, 0.f));
}

// Component d (0..3, a constant after unrolling) of a 16-byte vector.
__device__ __forceinline__ uint32_t& u4ref(uint4& v, int d) {
  return d == 0 ? v.x : (d == 1 ? v.y : (d == 2 ? v.z : v.w));
}

// ----------------------------------------------------------------------
// Operand loaders.  R = rows of the panel (M or N extent of the tile).
// ----------------------------------------------------------------------

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

#if defined(__HIP_DEVICE_COMPILE__)
// Buffer resource over `bytes` bytes from the wave-uniform address `origin`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel_rsrc(const uint16_t* origin,
                                                             uint32_t bytes) {
  const uint64_t base = reinterpret_cast<uint64_t>(origin);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  void* src = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  // word 3 = 0x00020000: 32-bit data format, the raw-buffer setting
  return __builtin_amdgcn_make_buffer_rsrc(src, (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 16-byte load at byte offset voff + soff (soff wave-uniform) of the buffer
// `rs`.  Interior tiles load their panels this way: one resource per
// panel and k-step (scalar registers), a per-thread byte offset fixed for
// the whole kernel, and a uniform offset per vector, so a load is one
// instruction with no address arithmetic or bounds test in the loop.
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                            uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
#endif

// Operand contiguous along K: stored row r (an m or n index) holds k.
template <int R, int NTH = kThreads>
struct LoaderKMajor {
  static constexpr int L = R * 8 / NTH;  // 16-byte chunks per thread per k-step
  uint4 v[L];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ld, int r0,
                                       int Rt, int k0, int K, bool aligned, int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int q = tid + NTH * i;
      const int row = q >> 3, kc = q & 7;
      const int gr = r0 + row, gk = k0 + kc * 8;
      if (aligned && gr < Rt && gk + 8 <= K) {
        v[i] = *reinterpret_cast<const uint4*>(X + (int64_t)gr * ld + gk);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (gr < Rt) {
          const uint16_t* p = X + (int64_t)gr * ld;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gk + e < K) w[e >> 1] |= (uint32_t)p[gk + e] << ((e & 1) * 16);
        }
        v[i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  // Interior tiles (the whole panel inside X, 16-byte aligned, ld % 8 ==
  // 0, (R-1)*ld*2 < 2^32): vector i of thread t is row t/8 + i*NTH/8,
  // chunk t%8 of the k-step, at a fixed per-thread byte offset plus i rows.
  uint32_t voff, sstep;

  __device__ __forceinline__ void init_interior(int64_t ld, int tid) {
    voff = (uint32_t)(((int64_t)(tid >> 3) * ld + (tid & 7) * 8) * 2);
    sstep = (uint32_t)(ld * (NTH / 8) * 2);
  }

  __device__ __forceinline__ void load_interior(const uint16_t* X, int64_t ld, int r0, int k0,
                                                bool zero = false) {
    prep_interior(X, ld, r0, k0, zero);
#pragma unroll
    for (int i = 0; i < L; ++i) load_unit(i);
  }

  // The same loads one vector at a time (see LoaderMNMajor): zero
  // (uniform) gives the buffer an empty range, so the vectors read as 0.
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t rs;
#endif
  __device__ __forceinline__ void prep_interior(const uint16_t* X, int64_t ld, int r0, int k0,
                                                bool zero = false) {
#if defined(__HIP_DEVICE_COMPILE__)
    rs = panel_rsrc(X + (int64_t)r0 * ld + k0,
                    zero ? 0u : (uint32_t)(((int64_t)(R - 1) * ld + kBK) * 2));
#else
    (void)X, (void)ld, (void)r0, (void)k0, (void)zero;
#endif
  }
  __device__ __forceinline__ void load_unit(int i) {
#if defined(__HIP_DEVICE_COMPILE__)
    v[i] = buf_load16(rs, voff, i * sstep);
#else
    (void)i;
#endif
  }

  // cast every loaded element to e4m3fn (Q8 epilogues); zero fill stays 0
  __device__ __forceinline__ void quantize(float sc) {
#pragma unroll
    for (int i = 0; i < L; ++i) q8_vec(v[i], sc);
  }

  // A cross-entropy gradient with tokens along the rows (A 'N'): vector i
  // holds 8 vocabulary columns (k) of token row r0 + i*NTH/8 + tid/8.  The
  // scales and labels of a k-step are loaded with its panel (load_g) and
  // applied one vector at a time (rescale_one).
  float gs[L];
  int gl[L];
  __device__ __forceinline__ void load_g(const GemmParams& p, int r0, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int q = tid + NTH * i;
      g_params(p, r0 + (q >> 3), k0 + (q & 7) * 8, gs[i], gl[i]);
    }
  }
  __device__ __forceinline__ void rescale_one(int i) { g_vec(v[i], gs[i], gl[i]); }

  // The store as U units (one 16-byte LDS write each), so that they can be
  // spread between matrix-core instructions.
  static constexpr int U = L;
  __device__ __forceinline__ void store_unit(uint16_t* lds, int tid, int i) const {
    const int q = tid + NTH * i;
    const int row = q >> 3, kc = q & 7;
    *reinterpret_cast<uint4*>(lds + row * kBK + ((kc ^ swz(row)) << 3)) = v[i];
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int q = tid + NTH * i;
      const int row = q >> 3, kc = q & 7;
      *reinterpret_cast<uint4*>(lds + row * kBK + ((kc ^ swz(row)) << 3)) = v[i];
    }
  }
};

// Operand contiguous along M/N: stored row k holds the m (or n) index.
// Thread t owns k-group kb (L consecutive k) of mn-chunk mc (8 consecutive
// rows of the panel); it loads L 16-byte vectors (one per k) and
// transposes them into LDS rows.
template <int R, int NTH = kThreads>
struct LoaderMNMajor {
  static constexpr int L = R * 8 / NTH;  // k values per thread per k-step
  static constexpr int KBN = kBK / L; // k-groups per k-step
  uint4 v[L];

  // Thread -> (k-group, mn-chunk).  A load instruction covers whole
  // 128-byte lines either way; what differs is how many consecutive lanes
  // read consecutive bytes.  With each lane on its own k row the loads
  // crowded the texture unit's address queue, so lane quads take
  // consecutive mn-chunks and read 64 contiguous bytes: thread bits 0-1 are
  // the chunk's low bits, the next 3 (256-row panels, 8 k-groups) or 4
  // (128-row panels, 16 k-groups) bits the k-group, the rest the chunk's
  // high bits.  The cost is on the LDS side: the 8 lanes of a write group
  // land on fewer distinct swizzled chunks, a bank conflict, which measured
  // cheaper than either reading 32 bytes per lane pair without conflicts or
  // selecting a per-lane row order that removes them.  Other panel sizes:
  // the k-group varies fastest.
  static_assert(KBN != 8 || NTH == 256, "the quad mapping covers 8 k-groups x 32 chunks");
  static __device__ __forceinline__ int kb_of(int tid) {
    if constexpr (KBN == 8) return (tid >> 2) & 7;
    if constexpr (KBN == 16 && NTH == 256) return (tid >> 2) & 15;
    return tid % KBN;
  }
  static __device__ __forceinline__ int mc_of(int tid) {
    if constexpr (KBN == 8) return (tid & 3) | ((tid >> 5) << 2);
    if constexpr (KBN == 16 && NTH == 256) return (tid & 3) | ((tid >> 6) << 2);
    return tid / KBN;
  }
  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ld, int r0,
                                       int Rt, int k0, int K, bool aligned, int tid) {
    const int kb = kb_of(tid), mc = mc_of(tid);
    const int gr = r0 + mc * 8;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int gk = k0 + kb * L + j;
      if (aligned && gk < K && gr + 8 <= Rt) {
        v[j] = *reinterpret_cast<const uint4*>(X + (int64_t)gk * ld + gr);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (gk < K) {
          const uint16_t* p = X + (int64_t)gk * ld;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gr + e < Rt) w[e >> 1] |= (uint32_t)p[gr + e] << ((e & 1) * 16);
        }
        v[j] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  // Interior tiles (the whole panel inside X, 16-byte aligned, ld % 8 ==
  // 0): vector j of thread t is k row kb*L + j, rows mc*8 .. +7, at a fixed
  // per-thread byte offset plus j rows of X.
  uint32_t voff, sstep;

  __device__ __forceinline__ void init_interior(int64_t ld, int tid) {
    const int kb = kb_of(tid), mc = mc_of(tid);
    voff = (uint32_t)(((int64_t)kb * L * ld + mc * 8) * 2);
    sstep = (uint32_t)(ld * 2);
  }

  // zero (uniform): an empty buffer range, so the vectors read as 0.
  __device__ __forceinline__ void load_interior(const uint16_t* X, int64_t ld, int r0, int k0,
                                                bool zero = false) {
    prep_interior(X, ld, r0, k0, zero);
#pragma unroll
    for (int j = 0; j < L; ++j) load_unit(j);
  }

  // The same loads one vector at a time, so that a loop can spread them
  // between matrix-core instructions: prep_interior makes the panel's
  // buffer resource, load_unit(j) loads vector j.
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t rs;
#endif
  __device__ __forceinline__ void prep_interior(const uint16_t* X, int64_t ld, int r0, int k0,
                                                bool zero = false) {
#if defined(__HIP_DEVICE_COMPILE__)
    rs = panel_rsrc(X + (int64_t)k0 * ld + r0,
                    zero ? 0u : (uint32_t)(((int64_t)(kBK - 1) * ld + R) * 2));
#else
    (void)X, (void)ld, (void)r0, (void)k0, (void)zero;
#endif
  }
  __device__ __forceinline__ void load_unit(int j) {
#if defined(__HIP_DEVICE_COMPILE__)
    v[j] = buf_load16(rs, voff, j * sstep);
#else
    (void)j;
#endif
  }

  __device__ __forceinline__ void quantize(float sc) {
#pragma unroll
    for (int j = 0; j < L; ++j) q8_vec(v[j], sc);
  }

  // A cross-entropy gradient stored [tokens][vocabulary] and read 'T' (the
  // GEMM's k is the token): vector j holds 8 vocabulary rows of token k.
  float gs[L];
  int gl[L];
  __device__ __forceinline__ void load_g(const GemmParams& p, int r0, int k0, int tid) {
    const int kb = kb_of(tid), mc = mc_of(tid);
#pragma unroll
    for (int j = 0; j < L; ++j) g_params(p, k0 + kb * L + j, r0 + mc * 8, gs[j], gl[j]);
  }
  __device__ __forceinline__ void rescale_one(int j) { g_vec(v[j], gs[j], gl[j]); }

  __device__ __forceinline__ uint32_t elem(int j, int i) const {
    return (u4comp(v[j], i >> 1) >> ((i & 1) * 16)) & 0xffffu;
  }

  // Element i of vectors j and j+1 as one dword (j's in the low half): one
  // byte permute of the dwords holding them.
  __device__ __forceinline__ uint32_t pair(int j, int i) const {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_perm(u4comp(v[j + 1], i >> 1), u4comp(v[j], i >> 1),
                                 (i & 1) ? 0x07060302u : 0x05040100u);
#else
    return elem(j, i) | (elem(j + 1, i) << 16);
#endif
  }

  // The store as U units (row i of the thread's 8 rows: the transposed
  // element i of every vector, one LDS write), so that they can be spread
  // between matrix-core instructions.
  static constexpr int U = 8;
  __device__ __forceinline__ void store_unit(uint16_t* lds, int tid, int i) const {
    const int kb = kb_of(tid), mc = mc_of(tid);
    const int row = mc * 8 + i;
    uint16_t* dst = lds + row * kBK;
    if constexpr (L == 8) {
      uint4 o;
      o.x = pair(0, i);
      o.y = pair(2, i);
      o.z = pair(4, i);
      o.w = pair(6, i);
      *reinterpret_cast<uint4*>(dst + ((kb ^ swz(row)) << 3)) = o;
    } else if constexpr (L == 4) {
      uint2 o;
      o.x = pair(0, i);
      o.y = pair(2, i);
      *reinterpret_cast<uint2*>(dst + (((kb >> 1) ^ swz(row)) << 3) + (kb & 1) * 4) = o;
    } else {
      static_assert(L == 2, "panel rows must be 64, 128 or 256");
      const uint32_t o = pair(0, i);
      *reinterpret_cast<uint32_t*>(dst + (((kb >> 2) ^ swz(row)) << 3) + (kb & 3) * 2) = o;
    }
  }

  // store_unit from the thread's unit-0 byte offset off0 (256-row panels):
  // row mc*8 + i has the swizzle swz(mc*8) ^ (i/2), so unit i sits at byte
  // (off0 ^ (i/2 << 4)) + 128 i -- one register for the eight units and an
  // XOR each, where store_unit's addresses take four registers.
  __device__ __forceinline__ uint32_t unit0_offset(int tid) const {
    const int kb = kb_of(tid), mc = mc_of(tid);
    return (uint32_t)((mc * 8 * kBK + ((kb ^ swz(mc * 8)) << 3)) * 2);
  }
  __device__ __forceinline__ void store_unit_at(uint16_t* lds, uint32_t off0, int i) const {
    static_assert(L == 8, "256-row panels");
    uint4 o;
    o.x = pair(0, i);
    o.y = pair(2, i);
    o.z = pair(4, i);
    o.w = pair(6, i);
    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(lds) + ((off0 ^ ((i >> 1) << 4)) + i * 128)) =
        o;
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    const int kb = kb_of(tid), mc = mc_of(tid);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = mc * 8 + i;
      uint16_t* dst = lds + row * kBK;
      if constexpr (L == 8) {
        uint4 o;
        o.x = pair(0, i);
        o.y = pair(2, i);
        o.z = pair(4, i);
        o.w = pair(6, i);
        *reinterpret_cast<uint4*>(dst + ((kb ^ swz(row)) << 3)) = o;
      } else if constexpr (L == 4) {
        uint2 o;
        o.x = pair(0, i);
        o.y = pair(2, i);
        *reinterpret_cast<uint2*>(dst + (((kb >> 1) ^ swz(row)) << 3) + (kb & 1) * 4) = o;
      } else {
        static_assert(L == 2, "panel rows must be 64, 128 or 256");
        const uint32_t o = pair(0, i);
        *reinterpret_cast<uint32_t*>(dst + (((kb >> 2) ^ swz(row)) << 3) + (kb & 3) * 2) = o;
      }
    }
  }
};

template <bool KMAJOR, int R, int NTH = kThreads>
struct LoaderSel {
  using type = LoaderKMajor<R, NTH>;
};
template <int R, int NTH>
struct LoaderSel<false, R, NTH> {
  using type = LoaderMNMajor<R, NTH>;
};

// ----------------------------------------------------------------------
// Workgroup -> tile mapping.  Workgroups are dealt round-robin to the 8
// XCDs (workgroup b runs on XCD b % 8), each with its own L2.  The first
// 8*floor(W/8) workgroups are renumbered so XCD x gets a contiguous range
// of logical workgroups.  With K split into `split` chunks the logical
// order is chunk-major -- all tiles of chunk 0, then chunk 1 -- so an XCD
// holds one K chunk of a run of tiles and reads only that chunk of the
// operands shared along M or N (measured on the 768x5120x13824 NT GEMM:
// a quarter of the X traffic, 3% faster at the sustained clock).  Tiles
// are ordered in groups of `groupM` tile rows (column-major inside a
// group), so the tiles one XCD runs at the same time share A rows and B
// columns in its L2.
// ----------------------------------------------------------------------
__device__ __forceinline__ void xcd_remap(int bid, int W, int split, int& tile, int& ks) {
  const int per = W >> 3;
  int l = bid;
  if (bid < per * 8) l = (bid & 7) * per + (bid >> 3);
  const int ntiles = W / split;
  ks = l / ntiles;
  tile = l - ks * ntiles;
}

__device__ __forceinline__ void tile_coords(int t, int tilesM, int tilesN, int groupM, int& tm,
                                            int& tn) {
  const int gsz = groupM * tilesN;
  const int g = t / gsz, r = t - g * gsz;
  const int gm0 = g * groupM;
  const int gm = min(groupM, tilesM - gm0);
  tm = gm0 + r % gm;
  tn = r / gm;
}

__device__ __forceinline__ void map_tile(int bid, int tilesM, int tilesN, int groupM, int& tm,
                                         int& tn) {
  int tile, ks;
  xcd_remap(bid, tilesM * tilesN, 1, tile, ks);
  tile_coords(tile, tilesM, tilesN, groupM, tm, tn);
}

// ----------------------------------------------------------------------
// Direct global -> LDS panel copy (interior tiles of K-contiguous operands).
//
// One wave-wide 16-byte load with the LDS destination writes 64 x 16 B =
// 1 KB of LDS = 8 panel rows of 128 B, lane l landing at row l/8, physical
// chunk l%8 of that block.  Each lane therefore fetches the logical chunk
// (l%8) ^ swz(row) of its row, which produces exactly the swizzled image the
// register path writes.  No VGPRs hold the data and no LDS write
// instructions are issued.
// ----------------------------------------------------------------------
//
// The copies use the buffer form: a resource (base = the panel origin,
// range = the panel's byte extent) in scalar registers, a fixed 32-bit
// per-lane offset and a uniform scalar offset per block.  Measured in the
// two-stage loop, this beats the global form, which the compiler turns
// into a 64-bit per-lane address and a vector add per copy.  The range
// makes the hardware drop any access past the panel (reads return 0).
// The caller guarantees R * ld * 2 < 2^32 (ld < 2^23 for R = 256).
template <int R>
struct DmaPanel {
  static constexpr int PER_WAVE = R / 32;  // 1 KB blocks issued by each of the 4 waves
  static_assert(PER_WAVE % 2 == 0, "panel rows must be a multiple of 64");
  // Block j of this wave covers rows (wave*PER_WAVE + j)*8 .. +7; lane l
  // fetches row +l/8 at logical chunk (l%8) ^ swz(row).  swz(row) depends
  // on j only through j%2, so the per-lane byte offset of block j is
  // e[j%2] + j * 8 * ld * 2: two registers per panel, the rest is uniform.
  uint32_t e[2];
  uint32_t row8_bytes;  // 8 rows, in bytes (uniform)
  uint32_t extent;      // bytes from the origin to the end of the panel's last row chunk

  __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
    const int row0 = wave * PER_WAVE * 8 + (lane >> 3);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = (lane & 7) ^ swz(row0 + 8 * q);
      e[q] = (uint32_t)(((int64_t)row0 * ld + c * 8) * 2);
    }
    row8_bytes = (uint32_t)(ld * 16);
    extent = (uint32_t)(((int64_t)(R - 1) * ld + kBK) * 2);
  }

  // Copy 1 KB block j of this wave's share.  origin = &X[r0][k0] (row r0
  // of the tile, k-step k0) and panel are wave-uniform.  zero (uniform):
  // the buffer gets an empty range, so every lane reads 0 and the block
  // fills with zeros.
  __device__ __forceinline__ void issue_one(const uint16_t* origin, uint16_t* panel, int wave_u,
                                            int j, bool zero = false) const {
    const int blk = wave_u * PER_WAVE + j;
#if defined(__HIP_DEVICE_COMPILE__)
    // (device pass only: the host pass cannot form the LDS address-space
    // pointer and would silently drop the kernel's launch stub)
    const uint64_t base = reinterpret_cast<uint64_t>(origin);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    void* src = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    // word 3 = 0x00020000: 32-bit data format, the raw-buffer setting
    const int range = (int)__builtin_amdgcn_readfirstlane(extent);
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(src, (short)0, zero ? 0 : range, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(panel + blk * 512), 16, (int)e[j & 1],
        (int)__builtin_amdgcn_readfirstlane(j * row8_bytes), 0, 0);
#else
    (void)origin, (void)panel, (void)blk;
#endif
  }

  __device__ __forceinline__ void issue(const uint16_t* origin, uint16_t* panel, int wave_u,
                                        bool zero = false) const {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) issue_one(origin, panel, wave_u, j, zero);
  }
};

// ----------------------------------------------------------------------
// Scales and labels of a cross-entropy gradient finished on load in the
// two-set loop.  Each wave copies, straight into LDS words of its own, the
// words its own lanes apply: per k-step one 256-byte direct copy of scales
// (and, tokens along K, one of labels), issued just before the k-step's
// register set, so no barrier is needed: the loop reads a set's words only
// after an explicit wait for their copies (the compiler's own waits did not
// cover them; a full-size run read stale words).  The two register sets'
// words sit in two separate LDS arrays (buf0, buf1), and AK's labels in a
// third: with one array, the compiler made every read of one set's words
// wait for the other set's copies, issued a substep earlier.  Per wave and
// buffer: 64 scale words, then 64 label words.
//  - AK (gradient read 'N': tokens along M, vocabulary along K): thread t's
//    vectors are token rows t/8 + 32i; lane l of wave w stages row
//    8w + l/8 + 32(l%8), so each thread's 8 rows are 8 consecutive words.
//    A k-step is one 64-column chunk: one scale per row.  The rows'
//    labels are staged once.
//  - otherwise ('T': vocabulary along M, tokens along K): the lane-quad
//    mapping puts all of wave w's vectors in the tile's 64-row chunk w, so
//    the wave stages that chunk's scales of the k-step's 64 tokens and
//    their labels, word l for token l.
// ----------------------------------------------------------------------
template <bool AK>
struct GaStage {
  static constexpr int kBufWords = 4 * 128;  // one buffer array: 4 waves
  static constexpr int kLabWords = 4 * 64;   // AK's label array
  static constexpr int kCopies = AK ? 1 : 2;  // copies per k-step (vector-memory operations)
  uint32_t* area[2];  // this wave's words in buf0 / buf1 (wave-uniform)
  uint32_t* labf;     // AK: this wave's labels
  uint32_t voff;      // this lane's byte offset in a staged run

  __device__ __forceinline__ void init(uint32_t* buf0, uint32_t* buf1, uint32_t* labs, int wave_u,
                                       int lane) {
    area[0] = buf0 + wave_u * 128;
    area[1] = buf1 + wave_u * 128;
    labf = labs + wave_u * 64;
    voff = AK ? (uint32_t)((8 * wave_u + (lane >> 3) + 32 * (lane & 7)) * 4) : (uint32_t)(lane * 4);
  }

  // One 4-byte direct copy per lane from `origin` (wave-uniform) into `dst`;
  // zero: an empty range, so the words read 0.
  __device__ __forceinline__ void copy(const void* origin, uint32_t bytes, uint32_t* dst,
                                       bool zero) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint64_t base = reinterpret_cast<uint64_t>(origin);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    void* src = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(src, (short)0, zero ? 0 : (int)bytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 4,
                                             (int)voff, 0, 0, 0);
#else
    (void)origin, (void)bytes, (void)dst, (void)zero;
#endif
  }

  // The words of the k-step starting at column kg into buffer b.
  __device__ __forceinline__ void issue(const GemmParams& p, int m0, int kg, int b, bool zero,
                                        int wave_u) const {
    if constexpr (AK) {
      copy(p.gscale + (int64_t)(kg / kCeScaleCols) * p.gtok + m0, 256 * 4, area[b], zero);
    } else {
      copy(p.gscale + (int64_t)(m0 / kCeScaleCols + wave_u) * p.gtok + kg, 64 * 4, area[b],
           zero);
      copy(p.glabels + kg, 64 * 4, area[b] + 64, zero);
    }
  }
  // AK: the labels of the tile's 256 token rows, once.
  __device__ __forceinline__ void issue_labels(const GemmParams& p, int m0) const {
    copy(p.glabels + m0, 256 * 4, labf, false);
  }

  // Staged words of buffer b (this thread's 8 are idx0 .. idx0+7): the
  // labels, scales 2r and 2r+1, one label (a lane's own word idx = lane
  // holds the token it staged).
  __device__ __forceinline__ const uint32_t* lab_words(int b) const {
    return AK ? labf : area[b] + 64;
  }
  __device__ __forceinline__ void read_labels(int b, int idx0, int (&lab)[8]) const {
    const uint4* pl = reinterpret_cast<const uint4*>(lab_words(b) + idx0);
    const uint4 l0 = pl[0], l1 = pl[1];
    const uint32_t lw[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) lab[i] = (int)lw[i];
  }
  __device__ __forceinline__ void read_scale_pair(int b, int idx0, int r, float (&s)[8]) const {
    const uint2 q = *reinterpret_cast<const uint2*>(area[b] + idx0 + 2 * r);
    s[2 * r] = __uint_as_float(q.x);
    s[2 * r + 1] = __uint_as_float(q.y);
  }
  __device__ __forceinline__ int read_label(int b, int idx) const {
    return (int)lab_words(b)[idx];
  }
  __device__ __forceinline__ float read_scale(int b, int idx) const {
    return __uint_as_float(area[b][idx]);
  }
};

// Wait until every global -> LDS copy this wave issued has landed.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Operand fragments of k-substep s (k = 16s .. 16s+15) for this wave.
// a_base / b_base: element offset of the lane's first A / B row in a stage;
// xo[s]: swizzled element offset of the lane's 16-byte chunk in substep s.
// Successive 32-row blocks are 32 LDS rows (4 KB) apart: immediate offsets.
template <int FM, int FN>
__device__ __forceinline__ void read_frags(const uint16_t* st, int a_base, int b_base, int xo,
                                           bf16x8_t* af, bf16x8_t* bfr) {
  const uint16_t* pa = st + a_base + xo;
  const uint16_t* pb = st + b_base + xo;
#pragma unroll
  for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * kBK);
#pragma unroll
  for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(pb + j * 32 * kBK);
}

// One 32x32x16 MFMA.  SW = false: acc block (i,j) holds C[m][n] with the
// column n in the lane (l%32) and the row m across registers.  SW = true
// swaps the operands, so the block holds C^T: the row m in the lane and
// 16 columns per lane across registers (used by the cross-entropy epilogue,
// whose row reductions then stay in registers).  Each output element is the
// same dot product either way.
template <bool SW>
__device__ __forceinline__ f32x16_t mma(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  if constexpr (SW)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int FM, int FN, bool SW = false>
__device__ __forceinline__ void mfma_block(const bf16x8_t* af, const bf16x8_t* bfr,
                                           f32x16_t (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = mma<SW>(af[i], bfr[j], acc[i][j]);
}

// One k-substep without copies: MFMA q, then (first FM+FN slots) one
// fragment read of the next substep.
template <int FM, int FN, bool SW>
__device__ __forceinline__ void plain_substep(f32x16_t (&acc)[FM][FN], const bf16x8_t* fa,
                                              const bf16x8_t* fb, bf16x8_t* na, bf16x8_t* nb,
                                              const uint16_t* rd_stage, int a_base, int b_base,
                                              int xo) {
  const uint16_t* pa = rd_stage + a_base + xo;
  const uint16_t* pb = rd_stage + b_base + xo;
#pragma unroll
  for (int q = 0; q < FM * FN; ++q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = mma<SW>(fa[i], fb[j], acc[i][j]);
    if (q < FM) na[q] = *reinterpret_cast<const bf16x8_t*>(pa + q * 32 * kBK);
    else if (q < FM + FN) nb[q - FM] = *reinterpret_cast<const bf16x8_t*>(pb + (q - FM) * 32 * kBK);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One k-substep without copies whose slots also issue the loads of
// loaders la then lb (buffer resources already made), spread evenly: the
// register loops' loads of k-step kt+3, which issued all at once fill the
// address queue and hold up the matrix-core issue.
template <int FM, int FN, bool SW, typename LdA, typename LdB>
__device__ __forceinline__ void load2_substep(f32x16_t (&acc)[FM][FN], const bf16x8_t* fa,
                                              const bf16x8_t* fb, bf16x8_t* na, bf16x8_t* nb,
                                              const uint16_t* rd_stage, int a_base, int b_base,
                                              int xo, LdA& la, LdB& lb) {
  constexpr int SL = FM * FN, U = LdA::L + LdB::L;
  const uint16_t* pa = rd_stage + a_base + xo;
  const uint16_t* pb = rd_stage + b_base + xo;
#pragma unroll
  for (int q = 0; q < SL; ++q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = mma<SW>(fa[i], fb[j], acc[i][j]);
    if (q < FM) na[q] = *reinterpret_cast<const bf16x8_t*>(pa + q * 32 * kBK);
    else if (q < FM + FN) nb[q - FM] = *reinterpret_cast<const bf16x8_t*>(pb + (q - FM) * 32 * kBK);
    // units u with floor(u * SL / U) == q
#pragma unroll
    for (int u = (q * U + SL - 1) / SL; u < U && (u * SL) / U == q; ++u) {
      if (u < LdA::L)
        la.load_unit(u);
      else
        lb.load_unit(u - LdA::L);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One k-substep of the register path: MFMA q, one fragment read of the
// next substep (first FM+FN slots), and, when `st_on` is set, the LDS store
// units of loaders `la` then `lb` (the next k-step's operand panels, into
// `da` and `db`), spread evenly over the slots.  GA (A is a cross-entropy
// gradient finished on load): B's units go first, and A's vectors are
// transformed one per slot in the slots before A's first unit, as late as
// possible after their loads were issued.
template <int FM, int FN, bool SW, bool GA = false, typename LdA, typename LdB>
__device__ __forceinline__ void store2_substep(f32x16_t (&acc)[FM][FN], const bf16x8_t* fa,
                                               const bf16x8_t* fb, bf16x8_t* na, bf16x8_t* nb,
                                               const uint16_t* rd_stage, int a_base, int b_base,
                                               int xo, LdA& la, const LdB& lb, uint16_t* da,
                                               uint16_t* db, int tid, bool st_on) {
  constexpr int SL = FM * FN, U = LdA::U + LdB::U;
  // GA: the slot of A's first store unit; A's L vectors are transformed in
  // the slots before it (all in slot 0 when it is slot 0)
  constexpr int A0 = GA ? (LdB::U * SL) / U : 0;
  const uint16_t* pa = rd_stage + a_base + xo;
  const uint16_t* pb = rd_stage + b_base + xo;
#pragma unroll
  for (int q = 0; q < SL; ++q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = mma<SW>(fa[i], fb[j], acc[i][j]);
    if (q < FM) na[q] = *reinterpret_cast<const bf16x8_t*>(pa + q * 32 * kBK);
    else if (q < FM + FN) nb[q - FM] = *reinterpret_cast<const bf16x8_t*>(pb + (q - FM) * 32 * kBK);
    if (st_on) {
      if constexpr (GA) {
#pragma unroll
        for (int v = 0; v < LdA::L; ++v)
          if ((A0 > 0 ? (v * A0) / LdA::L : 0) == q) la.rescale_one(v);
      }
      // units u with floor(u * SL / U) == q (GA: B's units first)
#pragma unroll
      for (int u = (q * U + SL - 1) / SL; u < U && (u * SL) / U == q; ++u) {
        if constexpr (GA) {
          if (u < LdB::U) lb.store_unit(db, tid, u);
          else la.store_unit(da, tid, u - LdB::U);
        } else {
          if (u < LdA::U) la.store_unit(da, tid, u);
          else lb.store_unit(db, tid, u - LdA::U);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ----------------------------------------------------------------------
// Ring pipeline for interior tiles of K-contiguous operands.
//
// LDS holds S = ring_stages<BM,BN>() stages of 32 k each (A panel [BM][32]
// then B panel [BN][32] bf16, 64-byte rows of four 16-byte chunks).  Copies
// of stage kt+S-1 are issued while stage kt is multiplied, so a copy has S-1
// stages of matrix-core work to arrive; one barrier per stage.  Logical chunk c of row r sits
// at physical chunk c ^ ((r >> 2) & 3): sixteen lanes reading one logical
// chunk of 16 consecutive rows hit 16 distinct 16-byte bank groups, and
// every copy instruction writes 1 KB of LDS contiguously.
// ----------------------------------------------------------------------
constexpr int kRK = 32;
constexpr int kRingLdsBytes = 160 * 1024;  // the whole LDS of a compute unit
// Ring depth for a BM x BN tile: five 32-wide stages, or fewer if they do
// not fit.  (Measured on the 768x5120x13824 NT GEMM with 128x128 tiles:
// 5 stages beat 7 and 10 -- the deeper rings only add LDS footprint.)
template <int BM, int BN>
constexpr int ring_stages() {
  return kRingLdsBytes / ((BM + BN) * kRK * 2) > 5 ? 5 : kRingLdsBytes / ((BM + BN) * kRK * 2);
}

__device__ __forceinline__ int rswz(int row) { return (row >> 2) & 3; }

// s_waitcnt immediate: vmcnt(vm), lgkmcnt(lgkm), expcnt left open.
__host__ __device__ constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

template <int R>
struct RingDma {
  static constexpr int PER_WAVE = R / 64;  // 1 KB blocks (16 rows) per wave
  static_assert(PER_WAVE >= 1, "panel rows must be a multiple of 64");
  // Block j of this wave covers rows (wave*PER_WAVE + j)*16 .. +15; lane l
  // fetches row +l/4, logical chunk (l%4) ^ rswz(row).  rswz(row) is
  // (l/16)%4 for every block, so one per-lane offset serves all blocks.
  uint32_t e;
  int64_t row16_bytes;

  __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
    const int row0 = wave * PER_WAVE * 16 + (lane >> 2);
    const int c = (lane & 3) ^ rswz(row0);
    e = (uint32_t)(((int64_t)row0 * ld + c * 8) * 2);
    row16_bytes = ld * 32;
  }

  __device__ __forceinline__ void issue_one(const uint16_t* origin, uint16_t* panel, int wave_u,
                                            int j) const {
    const int blk = wave_u * PER_WAVE + j;
#if defined(__HIP_DEVICE_COMPILE__)
    const uint64_t base = reinterpret_cast<uint64_t>(origin) + (uint64_t)(j * row16_bytes);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    const char* src = reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
    __builtin_amdgcn_global_load_lds(src + e,
                                     (__attribute__((address_space(3))) void*)(panel + blk * 512),
                                     16, 0, 0);
#else
    (void)origin, (void)panel, (void)blk;
#endif
  }
};

// Ring staging of one operand, rows = its M or N extent R.  Only the
// K-contiguous form exists (A 'N', B 'T'): a stage is the panel [R rows]
// [32 k] copied by RingDma, and a lane's MFMA fragment (row l%32 of a
// 32-row block, k = 8h .. 8h+7 of the 16-k substep, h = l/32) is one
// 16-byte read.  (An MN-contiguous operand staged as k-rows and read with
// ds_read_b64_tr_b16 needs two 8-byte reads per fragment; measured on this
// chip, each costs about three times the issue time of a 16-byte read next
// to the MFMAs, which made that form slower than the register path that
// transposes while writing LDS, so MN-contiguous operands use the latter.)
template <bool KM, int R>
struct RingOp;

template <int R>
struct RingOp<true, R> {
  RingDma<R> dma;
  int f0, f1;  // element offset of the lane's fragment (block 0) in substeps 0 and 1

  __device__ __forceinline__ void init(int64_t ld, int wave, int lane, int half) {
    dma.init(ld, wave, lane);
    const int h = lane >> 5, lc = lane & 31;
    const int base = (half * (R / 2) + lc) * kRK;
    f0 = base + (((0 + h) ^ rswz(lc)) << 3);
    f1 = base + (((2 + h) ^ rswz(lc)) << 3);
  }
  __device__ static const uint16_t* origin(const uint16_t* X, int64_t ld, int r0, int k0) {
    return X + (int64_t)r0 * ld + k0;
  }
  __device__ static int64_t kstep(int64_t, int kk) { return kk; }
  __device__ __forceinline__ void issue_one(const uint16_t* o, uint16_t* panel, int wave_u,
                                            int j) const {
    dma.issue_one(o, panel, wave_u, j);
  }
  template <int S>
  __device__ __forceinline__ bf16x8_t frag(const uint16_t* panel, int i) const {
    return *reinterpret_cast<const bf16x8_t*>(panel + (S == 0 ? f0 : f1) + i * 32 * kRK);
  }
};

// One 16-k substep of the ring loop as FM*FN issue slots: MFMA q, then the
// side work of slot q -- the fragment reads of substep RS of the panel
// stage `ra_st`/`rb_st` (first FM+FN slots) and, evenly spread over the
// slots, half HALF of the stage's global->LDS copies.  Spreading the copies
// over both substeps keeps their issue rate below what the texture path
// drains, so a wave never stalls on a full copy queue while its matrix core
// idles.
template <int FM, int FN, int NA, int NB, int BM, int HALF, int RS, bool AK, bool BK, int BN,
          bool SW = false>
__device__ __forceinline__ void ring_substep(f32x16_t (&acc)[FM][FN], const bf16x8_t* fa,
                                             const bf16x8_t* fb, bf16x8_t* na, bf16x8_t* nb,
                                             const RingOp<AK, BM>& ra, const uint16_t* ra_st,
                                             const RingOp<BK, BN>& rb, const uint16_t* rb_st,
                                             const uint16_t* oa, const uint16_t* ob, uint16_t* dst,
                                             int wave_u) {
  constexpr int RA = BM * kRK;
  constexpr int H = (NA + NB) / 2;  // copies per substep
  static_assert((NA + NB) % 2 == 0, "copies split evenly over two substeps");
  constexpr int STEP = (FM * FN) / H > 0 ? (FM * FN) / H : 1;
#pragma unroll
  for (int q = 0; q < FM * FN; ++q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = mma<SW>(fa[i], fb[j], acc[i][j]);
    // (the MFMA is issued before the slot's reads, so the wait for its own
    // operands never covers the reads issued after it)
    __builtin_amdgcn_sched_barrier(0);
    if (q < FM) na[q] = ra.template frag<RS>(ra_st, q);
    else if (q < FM + FN) nb[q - FM] = rb.template frag<RS>(rb_st, q - FM);
    if (q % STEP == 0 && q / STEP < H) {
      const int n = HALF * H + q / STEP;
      if (n < NA) ra.issue_one(oa, dst, wave_u, n);
      else rb.issue_one(ob, dst + RA, wave_u, n - NA);
    }
    if constexpr (STEP == 1 && FM * FN < H) {
      // more copies than slots: issue the rest with the last slot
      if (q == FM * FN - 1) {
#pragma unroll
        for (int c = FM * FN; c < H; ++c) {
          const int n = HALF * H + c;
          if (n < NA) ra.issue_one(oa, dst, wave_u, n);
          else rb.issue_one(ob, dst + RA, wave_u, n - NA);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// k range [k0, k0 + nk * kRK).
template <int BM, int BN, int FM, int FN, bool AK, bool BK, bool SW = false>
__device__ __forceinline__ void ring_mainloop(const GemmParams& p, int m0, int n0, int k0, int nk,
                                              uint16_t* lds, int wave, int lane, int wm, int wn,
                                              f32x16_t (&acc)[FM][FN]) {
  constexpr int RA = BM * kRK, RST = (BM + BN) * kRK, S = ring_stages<BM, BN>();
  constexpr int NA = BM / 64, NB = BN / 64;   // copies per wave per stage
  static_assert(S >= 3, "the ring needs three stages");
  // Prologue: stage 0 landed once at most S-2 later stages are in flight.
  // In the loop, at the wait of iteration kt (after its first substep) the
  // copies issued after stage kt+1's are stages kt+2 .. kt+S-2 and the
  // first half of stage kt+S-1.
  constexpr int WAIT_FIRST = waitcnt_imm((NA + NB) * (S - 2), 0);
  constexpr int WAIT_NEXT = waitcnt_imm((NA + NB) * (S - 3) + (NA + NB) / 2, 0);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  RingOp<AK, BM> ra;
  RingOp<BK, BN> rb;
  ra.init(p.lda, wave, lane, wm);
  rb.init(p.ldb, wave, lane, wn);
  const uint16_t* oa = RingOp<AK, BM>::origin(p.A, p.lda, m0, k0);
  const uint16_t* ob = RingOp<BK, BN>::origin(p.B, p.ldb, n0, k0);

  // Prologue: stages 0 .. S-2.  Stages past the end of K re-read stage 0
  // into slots that are never multiplied, which keeps the number of copies
  // in flight (and so the vmcnt waits) uniform.
#pragma unroll
  for (int g = 0; g < S - 1; ++g) {
    const int kk = (g < nk ? g : 0) * kRK;
    const uint16_t* sa = oa + RingOp<AK, BM>::kstep(p.lda, kk);
    const uint16_t* sb = ob + RingOp<BK, BN>::kstep(p.ldb, kk);
#pragma unroll
    for (int j = 0; j < NA; ++j) ra.issue_one(sa, lds + g * RST, wave_u, j);
#pragma unroll
    for (int j = 0; j < NB; ++j) rb.issue_one(sb, lds + g * RST + RA, wave_u, j);
  }
  __builtin_amdgcn_s_waitcnt(WAIT_FIRST);
  __builtin_amdgcn_s_barrier();
  bf16x8_t fa[2][FM], fb[2][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) fa[0][i] = ra.template frag<0>(lds, i);
#pragma unroll
  for (int j = 0; j < FN; ++j) fb[0][j] = rb.template frag<0>(lds + RA, j);

  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int nxt = cur + 1 == S ? 0 : cur + 1;
    const int slot = cur == 0 ? S - 1 : cur - 1;  // freed by stage kt-1
    const int kd = kt + S - 1;
    const int kk = (kd < nk ? kd : 0) * kRK;
    const uint16_t* sa = oa + RingOp<AK, BM>::kstep(p.lda, kk);
    const uint16_t* sb = ob + RingOp<BK, BN>::kstep(p.ldb, kk);
    const uint16_t* st = lds + cur * RST;
    __builtin_amdgcn_sched_barrier(0);
    ring_substep<FM, FN, NA, NB, BM, 0, 1, AK, BK, BN, SW>(acc, fa[0], fb[0], fa[1], fb[1], ra, st,
                                                          rb, st + RA, sa, sb, lds + slot * RST,
                                                          wave_u);
    // Stage kt+1 landed (own copies: vmcnt; everyone's: the barrier), and
    // every wave finished reading stage kt (lgkmcnt), which the copies of
    // the next iteration overwrite.
    __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* sn = lds + nxt * RST;
    ring_substep<FM, FN, NA, NB, BM, 1, 0, AK, BK, BN, SW>(acc, fa[1], fb[1], fa[0], fb[0], ra, sn,
                                                          rb, sn + RA, sa, sb, lds + slot * RST,
                                                          wave_u);
    cur = nxt;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));  // the trailing re-reads
  __builtin_amdgcn_s_barrier();
}

// ----------------------------------------------------------------------
// Epilogues.  Accumulator layout of v_mfma_f32_32x32x16: lane l, register r
// holds row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of its 32x32 block.
// A wave owns rows m0+wr0 .. +32*FM and columns n0+wc0 .. +32*FN.
// No epilogue touches LDS.
// ----------------------------------------------------------------------
// Column offset of register r of accumulator block j from the lane's first
// column, in the cross-entropy's transposed accumulators.
__device__ __forceinline__ int ce_cofs(int j, int r) { return j * 32 + 8 * (r >> 2) + (r & 3); }

// exp(y - m) as 2^((y - m) * log2 e) on the hardware exp2, which returns 0
// where the result would be subnormal: such terms lie below 2^-126 of a
// block sum that holds at least 1 (the max's own term).
__device__ __forceinline__ float ce_exp(float y, float m) {
  return __builtin_amdgcn_exp2f((y - m) * kLog2e);
}

// Cross-entropy of one row block of transposed accumulators (the 16*FN
// columns of row `row` that this lane holds, register r of block j at
// column cl + ce_cofs(j, r); the other half of the wave's columns of the
// row sit in lane l^32): the block max and the block sum of exp(y - max)
// into the partial tables, and the label logit if the label's column is
// among them.  Returns the max the exponentials were taken against.
// EDGE: some of the lane's columns lie at or past N (only in the last
// column of tiles); they read as -inf, so that the max and the sum take no
// term from them (exp of -inf is 0).
template <bool EDGE, int FN>
__device__ __forceinline__ float ce_row_block(const GemmParams& p, const f32x16_t (&acc)[FN],
                                              int row, int label, int cl, int h, int64_t pbase) {
  f32x16_t v[FN];
  if constexpr (EDGE) {
    // the empty asm makes the limit opaque per row block, so that the 16*FN
    // compares are made here, each used once, and not hoisted and held
    // across the row blocks
    int lim = p.N - cl;
    asm volatile("" : "+v"(lim));
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) v[j][r] = ce_cofs(j, r) < lim ? acc[j][r] : -INFINITY;
  }
  auto y = [&](int j, int r) {
    if constexpr (EDGE) return v[j][r];
    return acc[j][r];
  };
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, y(j, r));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  // a block with no column inside N: its sum is 0 (not exp(-inf + inf))
  const float mref = mx == -INFINITY ? 0.f : mx;
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += ce_exp(y(j, r), mref);
  sum += __shfl_xor(sum, 32, 64);
  // the label's offset from the lane's first column; the lane holds it if
  // it falls in one of the lane's 4-column groups (bit 2 clear)
  const int c = label - cl;
  const bool hit = c >= 0 && c < 32 * FN && (c & 4) == 0;
  if (__builtin_amdgcn_ballot_w64(hit)) {  // most row blocks hold no label
    float ylab = 0.f;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) ylab = c == ce_cofs(j, r) ? acc[j][r] : ylab;
    if (hit && row < p.M) p.ylabel[row] = ylab;
  }
  if (h == 0 && row < p.M) {
    p.part_m[pbase + row] = mx;
    p.part_s[pbase + row] = sum;
  }
  return mref;
}

template <int EPI, int FM, int FN, bool SW = false>
__device__ __forceinline__ void epilogue(const GemmParams& p, f32x16_t (&acc)[FM][FN], int m0,
                                         int n0, int wr0, int wc0, int pcol, int lane) {
  const int h = lane >> 5, lc = lane & 31;
  // (Q8, OS: the sum times the output scale, one fp32 multiply)
  constexpr bool OS = EPI == kEpiQ8Bf16 || EPI == kEpiQ8F32 || EPI == kEpiOsBf16 ||
                      EPI == kEpiOsF32;
  constexpr bool GS = EPI == kEpiGStoreBf16 || EPI == kEpiGStoreF32;
  if constexpr (EPI == kEpiStoreBf16 || EPI == kEpiStoreF32 || OS || GS) {
    float os = 1.f;
    if constexpr (OS) os = p.qscales[2];
    // One output row at a time: its address is formed once, and the FN
    // column blocks of the row are immediate offsets from it.  A wave whose
    // whole block lies inside C stores without bounds tests.
    const int col0 = n0 + wc0 + lc;
    const bool full = m0 + wr0 + 32 * FM <= p.M && n0 + wc0 + 32 * FN <= p.N;
    auto put = [&](int64_t off, float v) __attribute__((always_inline)) {
      if constexpr (OS) v = __fmul_rn(v, os);
      if constexpr (EPI == kEpiStoreBf16 || EPI == kEpiQ8Bf16 || EPI == kEpiOsBf16 ||
                    EPI == kEpiGStoreBf16)
        reinterpret_cast<uint16_t*>(p.C)[off] = to_bf16(v);
      else
        reinterpret_cast<float*>(p.C)[off] = v;
    };
    if (full) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wr0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const int64_t off = (int64_t)row * p.ldc + col0;
#pragma unroll
          for (int j = 0; j < FN; ++j) put(off + j * 32, acc[i][j][r]);
        }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wr0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row >= p.M) continue;
          const int64_t off = (int64_t)row * p.ldc + col0;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (col0 + j * 32 < p.N) put(off + j * 32, acc[i][j][r]);
        }
    }
  } else {
    static_assert(SW, "the cross-entropy epilogue reads transposed accumulators");
    // Cross-entropy on transposed accumulators: block (i,j), register r of
    // lane l holds C[row i*32 + l%32][col j*32 + 8*(r/4) + 4*(l/32) + r%4].
    // A lane owns 16*FN columns of one row; the other half of the wave's
    // columns of that row sit in lane l^32.  Per row: block max, block sum
    // of exp(y - max), the label logit if its column is in the block, and
    // optionally exp(y - block max) into the gradient buffer (4 consecutive
    // columns per 8-byte store).  The logits themselves are not stored.
    const int64_t pbase = (int64_t)pcol * p.M;
    const bool vec8 = p.grad && (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(p.grad) & 7) == 0;
    // column of this lane's register 0 of block 0
    const int cl = n0 + wc0 + 4 * h;
    // the wave's columns reach past N only in the last column of tiles
    const bool edge = __builtin_amdgcn_readfirstlane(n0 + wc0 + 32 * FN > p.N ? 1 : 0) != 0;
    float rmax[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = m0 + wr0 + i * 32 + lc;
      const int label = row < p.M ? p.labels[row] : -1;  // (lanes l, l^32 share a row)
      if (edge)
        rmax[i] = ce_row_block<true>(p, acc[i], row, label, cl, h, pbase);
      else
        rmax[i] = ce_row_block<false>(p, acc[i], row, label, cl, h, pbase);
      // one row block at a time: keeps only its 16*FN values live
      __builtin_amdgcn_sched_barrier(0);
    }
    if (p.grad) {
      // exp(y - block max) into the gradient buffer, 4 consecutive columns
      // per 8-byte store (a pass of its own, so that the stores do not
      // lengthen the live ranges of the reductions above)
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = m0 + wr0 + i * 32 + lc;
        if (row >= p.M) continue;
        uint16_t* grow = p.grad + (int64_t)row * p.ldc + cl;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int co = ce_cofs(j, 4 * a);
            float e[4];
#pragma unroll
            for (int b = 0; b < 4; ++b)
              e[b] = ce_exp(acc[i][j][4 * a + b], rmax[i]);
            if (vec8 && cl + co + 4 <= p.N) {
              *reinterpret_cast<uint2*>(grow + co) =
                  make_uint2(pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]));
            } else {
#pragma unroll
              for (int b = 0; b < 4; ++b)
                if (cl + co + b < p.N) grow[co + b] = to_bf16(e[b]);
            }
          }
      }
    }
  }
}

// ----------------------------------------------------------------------
// Three-buffer pipeline for 256x256 interior tiles of K-contiguous operands
// (k-step 64, four substeps, one barrier per k-step).  LDS holds two A
// panels and three B panels of 32 KB each, the whole 160 KB.  B -- the
// weight, the operand that streams from HBM -- is copied a k-step earlier
// than A: the copies of B for k-step kt+2 go out in the first substep of
// kt, into the buffer k-step kt-1 used, and have about six substeps to
// land; the copies of A for k-step kt+2 go out after the barrier of kt, in
// its last substep, into the buffer kt used.  Each substep that copies
// issues one copy every other MFMA.  At the barrier of k-step kt only the
// copies of B for kt+2 may still be in flight, so one wait covers both
// operands of kt+1.
// ----------------------------------------------------------------------

// One substep: MFMA q, one fragment read of the next substep (first FM+FN
// slots, from pa / pb), and, when `cp` is set, this wave's copies of one
// panel (d, origin o, into dst), spread evenly over the slots.
// plain_substep with hook(q) run in slot q (side work spread between the
// matrix-core instructions).
template <int FM, int FN, bool SW, typename H>
__device__ __forceinline__ void hook_substep(f32x16_t (&acc)[FM][FN], const bf16x8_t* fa,
                                             const bf16x8_t* fb, bf16x8_t* na, bf16x8_t* nb,
                                             const uint16_t* rd_stage, int a_base, int b_base,
                                             int xo, H&& hook) {
  const uint16_t* pa = rd_stage + a_base + xo;
  const uint16_t* pb = rd_stage + b_base + xo;
#pragma unroll
  for (int q = 0; q < FM * FN; ++q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = mma<SW>(fa[i], fb[j], acc[i][j]);
    if (q < FM) na[q] = *reinterpret_cast<const bf16x8_t*>(pa + q * 32 * kBK);
    else if (q < FM + FN) nb[q - FM] = *reinterpret_cast<const bf16x8_t*>(pb + (q - FM) * 32 * kBK);
    hook(q);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int FM, int FN, int R, bool SW>
__device__ __forceinline__ void copy_substep(f32x16_t (&acc)[FM][FN], const bf16x8_t* fa,
                                             const bf16x8_t* fb, bf16x8_t* na, bf16x8_t* nb,
                                             const uint16_t* pa, const uint16_t* pb, bool cp,
                                             const DmaPanel<R>& d, const uint16_t* o,
                                             uint16_t* dst, int wave_u) {
  constexpr int NCP = DmaPanel<R>::PER_WAVE;
  constexpr int SL = FM * FN;
#pragma unroll
  for (int q = 0; q < FM * FN; ++q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = mma<SW>(fa[i], fb[j], acc[i][j]);
    if (q < FM) na[q] = *reinterpret_cast<const bf16x8_t*>(pa + q * 32 * kBK);
    else if (q < FM + FN) nb[q - FM] = *reinterpret_cast<const bf16x8_t*>(pb + (q - FM) * 32 * kBK);
    // copy c goes with slot floor(c * SL / NCP): evenly spread whatever the
    // counts (one every other slot for a 256x256 tile)
    if (cp) {
#pragma unroll
      for (int c = 0; c < NCP; ++c)
        if ((c * SL) / NCP == q) d.issue_one(o, dst, wave_u, c);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// k-steps [k0/64, k0/64 + nk).  a_base / b_local: element offsets of the
// lane's first A / B fragment row inside a panel buffer.
template <int BM, int BN, int FM, int FN, bool SW = false>
__device__ __forceinline__ void dma3_mainloop(const GemmParams& p, int m0, int n0, int k0, int nk,
                                              uint16_t* lds, int wave, int lane, int a_base,
                                              int b_local, const int* xo,
                                              f32x16_t (&acc)[FM][FN]) {
  constexpr int SA = BM * kBK, SB = BN * kBK;
  constexpr int NA = DmaPanel<BM>::PER_WAVE, NB = DmaPanel<BN>::PER_WAVE;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  DmaPanel<BM> da;
  DmaPanel<BN> db;
  da.init(p.lda, wave, lane);
  db.init(p.ldb, wave, lane);
  const uint16_t* oa = p.A + (int64_t)m0 * p.lda + k0;
  const uint16_t* ob = p.B + (int64_t)n0 * p.ldb + k0;
  uint16_t* const abuf = lds;            // two A panels
  uint16_t* const bbuf = lds + 2 * SA;   // three B panels
  // k-steps past the end re-read k-step 0 into a buffer that is never
  // multiplied, which keeps the copy counts, and so the waits, uniform
  auto kof = [nk](int t) { return (t < nk ? t : 0) * kBK; };
  // Prologue: A(0), B(0), B(1), A(1), in this order.
  da.issue(oa + kof(0), abuf, wave_u);
  db.issue(ob + kof(0), bbuf, wave_u);
  db.issue(ob + kof(1), bbuf + SB, wave_u);
  da.issue(oa + kof(1), abuf + SA, wave_u);
  // A(0), B(0) landed (own copies; other waves: the barrier).  A raw
  // barrier: the compiler's __syncthreads would also wait for B(1), A(1).
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(NA + NB, 0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_t fa[2][FM], fb[2][FN];
  read_frags<FM, FN>(abuf, a_base, b_local + 2 * SA, xo[0], fa[0], fb[0]);
  int b3 = 0;  // kt % 3
  for (int kt = 0; kt < nk; ++kt) {
    const int b3n = b3 == 2 ? 0 : b3 + 1;  // (kt + 1) % 3
    const int b3p = b3 == 0 ? 2 : b3 - 1;  // (kt + 2) % 3, the buffer k-step kt-1 used
    const uint16_t* ac = abuf + (kt & 1) * SA + a_base;
    const uint16_t* bc = bbuf + b3 * SB + b_local;
    const uint16_t* an = abuf + ((kt + 1) & 1) * SA + a_base;
    const uint16_t* bn = bbuf + b3n * SB + b_local;
    __builtin_amdgcn_sched_barrier(0);
    copy_substep<FM, FN, BN, SW>(acc, fa[0], fb[0], fa[1], fb[1], ac + xo[1], bc + xo[1], true, db,
                                 ob + kof(kt + 2), bbuf + b3p * SB, wave_u);
    copy_substep<FM, FN, BN, SW>(acc, fa[1], fb[1], fa[0], fb[0], ac + xo[2], bc + xo[2], false,
                                 db, ob, bbuf, wave_u);
    copy_substep<FM, FN, BN, SW>(acc, fa[0], fb[0], fa[1], fb[1], ac + xo[3], bc + xo[3], false,
                                 db, ob, bbuf, wave_u);
    // A(kt+1) and B(kt+1) landed (own copies: all but the NB just issued;
    // other waves: the barrier), and every LDS read of this wave is done
    // (lgkmcnt 0), so after the barrier no wave reads A(kt) any more.  A
    // raw barrier: the compiler's __syncthreads would also wait for the
    // copies of B(kt+2).
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(NB, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    copy_substep<FM, FN, BM, SW>(acc, fa[1], fb[1], fa[0], fb[0], an + xo[0], bn + xo[0], true, da,
                                 oa + kof(kt + 2), abuf + (kt & 1) * SA, wave_u);
    b3 = b3n;
  }
  // the trailing re-reads must land before the LDS is reused or released
  wait_dma();
  __syncthreads();
}

// ----------------------------------------------------------------------
// Mixed staging for interior 256x256 tiles with exactly one K-contiguous
// operand (NN: A; TT: B).  That operand (D) goes global -> LDS with the
// direct copies into three panel buffers, the copies of k-step kt+2 issued
// during substep 0 of kt, as in the three-buffer loop.  The other operand
// (G, contiguous along M or N) is loaded into registers in two sets: the
// set holding k-step kt+1 is transposed into one of two LDS panels during
// substep 2 of kt and, after the barrier, receives k-step kt+3 -- seven
// substeps of matrix-core work for its loads to arrive, where a single set
// leaves three.  LDS: 3 + 2 panels of 32 KB.
// ----------------------------------------------------------------------

// One substep of the mixed loop: MFMA q, one fragment read of the next
// substep (first FM+FN slots), this wave's copies of one D panel when `cp`
// (one every SL/NCP slots), and the G set's LDS store units when `st`
// (one every SL/U slots).
template <int FM, int FN, int R, bool SW, typename LG>
__device__ __forceinline__ void mix_substep(f32x16_t (&acc)[FM][FN], const bf16x8_t* fa,
                                            const bf16x8_t* fb, bf16x8_t* na, bf16x8_t* nb,
                                            const uint16_t* pa, const uint16_t* pb, bool cp,
                                            const DmaPanel<R>& d, const uint16_t* o,
                                            uint16_t* ddst, int wave_u, bool st, LG& g,
                                            uint16_t* gdst, int tid, bool zero = false,
                                            bool ld = false) {
  constexpr int SL = FM * FN;
  constexpr int NCP = DmaPanel<R>::PER_WAVE;
  static_assert(SL % NCP == 0 && SL % LG::U == 0 && SL % LG::L == 0,
                "side work must divide the slots evenly");
#pragma unroll
  for (int q = 0; q < SL; ++q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = mma<SW>(fa[i], fb[j], acc[i][j]);
    if (q < FM) na[q] = *reinterpret_cast<const bf16x8_t*>(pa + q * 32 * kBK);
    else if (q < FM + FN) nb[q - FM] = *reinterpret_cast<const bf16x8_t*>(pb + (q - FM) * 32 * kBK);
    if (cp && q % (SL / NCP) == 0) d.issue_one(o, ddst, wave_u, q / (SL / NCP), zero);
    if (st && q % (SL / LG::U) == 0) g.store_unit(gdst, tid, q / (SL / LG::U));
    if (ld && q % (SL / LG::L) == 0) g.load_unit(q / (SL / LG::L));
    __builtin_amdgcn_sched_barrier(0);
  }
}

// k-steps [k0/64, k0/64 + nk); AK: A is the K-contiguous operand (else B).
template <int BM, int BN, int FM, int FN, bool AK, bool SW>
__device__ __forceinline__ void mix_mainloop(const GemmParams& p, int m0, int n0, int k0, int nk,
                                             uint16_t* __restrict__ dbuf,
                                             uint16_t* __restrict__ gbuf, int tid, int wave,
                                             int lane, int a_base, int b_local, const int* xo,
                                             f32x16_t (&acc)[FM][FN]) {
  // dbuf: three D panels; gbuf: two G panels.  They do not overlap, and
  // saying so lets the compiler write G into LDS without first waiting for
  // every direct copy in flight (which only write D's panels).
  static_assert(BM == BN, "one panel size for both operands");
  constexpr int SP = BM * kBK;
  constexpr int ND = DmaPanel<BM>::PER_WAVE;
  using LG = LoaderMNMajor<BM>;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  DmaPanel<BM> dp;
  dp.init(AK ? p.lda : p.ldb, wave, lane);
  const uint16_t* od = AK ? p.A + (int64_t)m0 * p.lda + k0 : p.B + (int64_t)n0 * p.ldb + k0;
  const uint16_t* XG = AK ? p.B : p.A;
  const int64_t ldg = AK ? p.ldb : p.lda;
  const int rg0 = AK ? n0 : m0;
  LG g0, g1;
  g0.init_interior(ldg, tid);
  g1.init_interior(ldg, tid);
  // The loop runs an even number of k-steps, nke: with nk odd, k-step nk
  // is one of zeros (both operands' loads get an empty buffer range), which
  // adds exactly nothing to the sums.  A loop entered only from this
  // prologue and from its own back edge sees the loads in one order, so the
  // wait the compiler places before each register set's LDS stores waits
  // for that set alone, giving its loads seven substeps to arrive.  (An odd
  // k-step run outside the loop either merged two orders at the loop's
  // entry, whose wait then also covered the other set, or, after the loop,
  // made the register allocator spill the accumulators.)
  const int nke = nk + (nk & 1);
  // k-steps past nke re-read k-step 0 (never stored or multiplied), so
  // every k-step issues the same loads and the wait counts stay fixed
  auto kof = [nk](int t) { return (t < nk ? t : 0) * kBK; };
  auto zero = [nk, nke](int t) { return t == nk && nke != nk; };
  // fragment rows: A's panel base + a_base, B's + b_local
  auto pa_of = [&](uint16_t* d, uint16_t* g) { return (AK ? d : g) + a_base; };
  auto pb_of = [&](uint16_t* d, uint16_t* g) { return (AK ? g : d) + b_local; };
  // The step of k-step kt takes the set holding kt+1: g1 for even kt, g0
  // for odd.
  auto prologue = [&](LG& s0, LG& s1) __attribute__((always_inline)) {
    // s0 carries k-step 0, then k-step 2; s1 carries k-step 1.  The loads
    // leave in the loop's own order -- the set of k-step kt+1, then the
    // copies of D(kt+1), then the set of kt+2 -- so that the wait the
    // compiler places before each set's LDS stores, which must hold for
    // both the entry and the back edge of the loop, waits for that set
    // alone and not also for the other one.
    dp.issue(od + kof(0), dbuf, wave_u);
    s0.load_interior(XG, ldg, rg0, k0 + kof(0));
    s1.load_interior(XG, ldg, rg0, k0 + kof(1), zero(1));
    dp.issue(od + kof(1), dbuf + SP, wave_u, zero(1));
    s0.store(gbuf, tid);
    s0.load_interior(XG, ldg, rg0, k0 + kof(2), zero(2));
  };
  prologue(g0, g1);
  // D(0) landed (issued first; the rest may be in flight: G(0) done, G(1),
  // D(1), G(2)); the G(0) stores done; other waves: the barrier
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(ND + 2 * LG::L, 0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_t fa[2][FM], fb[2][FN];
  {
    const uint16_t* pa = pa_of(dbuf, gbuf) + xo[0];
    const uint16_t* pb = pb_of(dbuf, gbuf) + xo[0];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * kBK);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = *reinterpret_cast<const bf16x8_t*>(pb + j * 32 * kBK);
  }
  // k-step kt; g holds k-step kt+1 and then receives kt+3
  auto step = [&](LG& g, int kt) __attribute__((always_inline)) {
    const int d3 = kt % 3, d3n = (kt + 1) % 3, d3p = (kt + 2) % 3;
    uint16_t* dc = dbuf + d3 * SP;
    uint16_t* gc = gbuf + (kt & 1) * SP;
    uint16_t* dn = dbuf + d3n * SP;
    uint16_t* gn = gbuf + ((kt + 1) & 1) * SP;
    const uint16_t* pa = pa_of(dc, gc);
    const uint16_t* pb = pb_of(dc, gc);
    __builtin_amdgcn_sched_barrier(0);
    mix_substep<FM, FN, BM, SW>(acc, fa[0], fb[0], fa[1], fb[1], pa + xo[1], pb + xo[1], true, dp,
                                od + kof(kt + 2), dbuf + d3p * SP, wave_u, false, g, gn, tid,
                                zero(kt + 2));
    mix_substep<FM, FN, BM, SW>(acc, fa[1], fb[1], fa[0], fb[0], pa + xo[2], pb + xo[2], false,
                                dp, od, dbuf, wave_u, false, g, gn, tid);
    // (the set always holds a k-step -- past the end a re-read of k-step
    // 0 -- so its stores need no test: in the last k-step they fill a stage
    // that is never multiplied)
    mix_substep<FM, FN, BM, SW>(acc, fa[0], fb[0], fa[1], fb[1], pa + xo[3], pb + xo[3], false,
                                dp, od, dbuf, wave_u, true, g, gn, tid);
    // D(kt+1) landed (after its copies: G(kt+2)'s loads and D(kt+2)'s
    // copies), the G stores and this wave's fragment reads done; after the
    // barrier no wave reads D(kt) or G(kt) any more
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(LG::L + ND, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // G(kt+3)'s loads, one every SL/L slots of this substep (issued all at
    // once they fill the address queue and hold up the matrix-core issue)
    g.prep_interior(XG, ldg, rg0, k0 + kof(kt + 3), zero(kt + 3));
    mix_substep<FM, FN, BM, SW>(acc, fa[1], fb[1], fa[0], fb[0], pa_of(dn, gn) + xo[0],
                                pb_of(dn, gn) + xo[0], false, dp, od, dbuf, wave_u, false, g, gn,
                                tid, false, true);
  };
  // the body is two unconditional steps (a conditional second step, or a
  // second exit, merges two versions of the accumulators inside the loop,
  // which the register allocator does not keep in place)
  for (int kt = 0; kt < nke; kt += 2) {
    step(g1, kt);
    step(g0, kt + 1);
  }
  // the trailing loads must land before the LDS is reused or released
  wait_dma();
  __syncthreads();
}

// ----------------------------------------------------------------------
// Two register sets per operand, for interior 256x256 tiles with both
// operands contiguous along M or N (TN), which the direct copies cannot
// stage.  The sets holding k-step kt+1 are transposed into the other LDS
// stage during substep 2 of kt and, after the barrier, receive k-step
// kt+3: seven substeps for their loads to arrive, where one set per operand
// leaves three.
// GA: A is a cross-entropy gradient finished on load (K-contiguous when AK,
// so NN runs here too); its scales and labels come through GaStage, and
// the A vectors are transformed one dword per slot over substeps 0 to 2 of
// the k-step that stores them, before their LDS stores.
// ----------------------------------------------------------------------
// k-steps [k0/64, k0/64 + nk).
template <int BM, int BN, int FM, int FN, bool SW, bool AK = false, bool GA = false>
__device__ __forceinline__ void reg2_mainloop(const GemmParams& p, int m0, int n0, int k0, int nk,
                                              uint16_t* __restrict__ lds,
                                              uint32_t* __restrict__ gbuf0,
                                              uint32_t* __restrict__ gbuf1,
                                              uint32_t* __restrict__ glabs, int tid, int a_base,
                                              int b_base, const int* xo,
                                              f32x16_t (&acc)[FM][FN]) {
  using LA = typename LoaderSel<AK, BM>::type;
  using LB = LoaderMNMajor<BN>;
  static_assert(!AK || GA, "K-contiguous A takes this loop only as a gradient");
  static_assert(!GA || LA::L == 8, "the gradient transform covers 8 vectors per thread");
  // LDS: stage s holds A at s*SSTR and B BOFF after it.  GA: A of stages
  // 0 and 1, then B of stages 0 and 1, so that the two stages of a panel
  // lie 32 KB apart, within the LDS instructions' immediate offset, and the
  // LDS addresses of both stages share registers (the transform needs
  // them; the plain loop measured 2% faster with the stages 64 KB apart).
  static_assert(BM == BN, "one panel size");
  constexpr int SA = BM * kBK;
  constexpr int SSTR = GA ? SA : 2 * SA, BOFF = GA ? 2 * SA : SA;
  const int bb = b_base - SA + BOFF;  // B's fragment rows, from the stage's A panel
  LA a0, a1;
  LB b0, b1;
  a0.init_interior(p.lda, tid);
  a1.init_interior(p.lda, tid);
  b0.init_interior(p.ldb, tid);
  b1.init_interior(p.ldb, tid);
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  GaStage<AK> ga;
  // GA: this thread's first staged word; what its label offsets are
  // relative to (AK: the vector's first vocabulary column, less the
  // k-step's; else the vector's first vocabulary row); not AK, the first of
  // the wave's 64 vocabulary rows
  int ga_idx0 = 0, ga_rel0 = 0, ga_hb = 0;
  if constexpr (GA) {
    ga.init(gbuf0, gbuf1, glabs, wave_u, tid & 63);
    if constexpr (AK) {
      ga.issue_labels(p, m0);
      ga_idx0 = ((tid >> 3) & 7) * 8;
      ga_rel0 = 8 * (tid & 7);
    } else {
      ga_idx0 = LA::kb_of(tid) * 8;
      ga_rel0 = m0 + LA::mc_of(tid) * 8;
      ga_hb = m0 + 64 * wave_u;
    }
  }
  // An even number of k-steps, nke, with k-step nk of zeros when nk is odd
  // (see mix_mainloop: one order of loads at the loop's entry and back
  // edge, so each set's stores wait for that set alone).  k-steps past nke
  // re-read k-step 0 (never stored), keeping the loads of every k-step
  // alike.
  const int nke = nk + (nk & 1);
  auto kof = [nk](int t) { return (t < nk ? t : 0) * kBK; };
  // (GA: the k-step's staged words first, so the wait for the set covers
  // them; buffer = the set's index)
  auto load = [&](LA& a, LB& b, int t, int buf) __attribute__((always_inline)) {
    const bool zero = t == nk && nke != nk;
    if constexpr (GA) ga.issue(p, m0, k0 + kof(t), buf, zero, wave_u);
    a.load_interior(p.A, p.lda, m0, k0 + kof(t), zero);
    b.load_interior(p.B, p.ldb, n0, k0 + kof(t), zero);
  };
  // GA: what the staged labels of k-step t are offset by
  auto ga_rel = [&](int t) { return AK ? k0 + kof(t) + ga_rel0 : ga_rel0; };
  // GA: whether any lane of the wave has a label column among its vectors
  // of k-step t: each lane tests the label it staged against the wave's 64
  // columns (AK) or rows
  auto ga_hb_of = [&](int t) { return AK ? k0 + kof(t) : ga_hb; };
  auto ga_wave_hit = [](int own, int hb) __attribute__((always_inline)) {
    return __builtin_amdgcn_ballot_w64((unsigned)(own - hb) < 64u) != 0;
  };
  const uint32_t b_off0 = b0.unit0_offset(tid);
  // the sets for k-steps 0 / 2 and 1
  load(a0, b0, 0, 0);
  load(a1, b1, 1, 1);
  if constexpr (GA) {
    // (k-step 0's words: wait until at most k-step 1's copies and loads
    // are outstanding, so k-step 0's copies, and AK's labels issued before
    // them, have landed)
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(LA::L + LB::L + GaStage<AK>::kCopies, 15));
    float gsv[8];
    int glv[8];
    ga.read_labels(0, ga_idx0, glv);
#pragma unroll
    for (int r = 0; r < 4; ++r) ga.read_scale_pair(0, ga_idx0, r, gsv);
    const int r0 = ga_rel(0);
#pragma unroll
    for (int v = 0; v < 8; ++v) g_vec(a0.v[v], gsv[v], glv[v] - r0);
  }
  a0.store(lds, tid);
  b0.store(lds + BOFF, tid);
  load(a0, b0, 2, 0);
  __syncthreads();
  bf16x8_t fa[2][FM], fb[2][FN];
  read_frags<FM, FN>(lds, a_base, bb, xo[0], fa[0], fb[0]);
  // k-step kt; (a, b) hold k-step kt+1 and then receive kt+3
  auto step = [&](LA& a, LB& b, int kt, int buf) __attribute__((always_inline)) {
    const int cur = kt & 1;
    const uint16_t* st = lds + cur * SSTR;
    uint16_t* nx = lds + (cur ^ 1) * SSTR;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (GA) {
      // The transform of set a (k-step kt+1), one dword of a vector (two
      // elements, five vector instructions) per slot from slot 3 of
      // substep 0 to slot 2 of substep 2, with no branch per vector;
      // substep 2 then stores B's units first and A's last.  In a k-step where a
      // lane of the wave has a label column among its vectors (about one
      // in eight; each lane tests the label it staged against the wave's
      // 64 columns (AK) or rows), slot 2 instead applies the full form to
      // all eight vectors at once, and the spread dwords multiply by 1,
      // which leaves bf16 values as they are.  Scales are read two at a
      // time, two slots ahead, so few words are live.  The staged words
      // are read only after an explicit wait for their copies: the
      // vector-memory operations issued since are this set's loads and
      // k-step kt+2's copies and loads (the loop holds no other
      // vector-memory operation; the vectors' own waits are the
      // compiler's).
      const int r0 = ga_rel(kt + 1);
      float gsv[8];
      int own = 0;
      bool hit = false;
      uint32_t bo = b_off0;
      constexpr int SL = FM * FN, U = LA::U + LB::U;
      // P0: the first dword's slot; RA: how many slots ahead of its first
      // use a scale pair is read
      constexpr int P0 = 3, RA = 2;
      static_assert(P0 >= 3 && RA >= 1 && RA <= P0 && P0 + 31 < 2 * SL + LB::U,
                    "the label test and the scale reads precede the dwords, which end "
                    "before A's stores");
      auto slot = [&](int g) __attribute__((always_inline)) {
        if (g == 0) {
          __builtin_amdgcn_s_waitcnt(
              waitcnt_imm(2 * (LA::L + LB::L) + GaStage<AK>::kCopies, 15));
          own = ga.read_label(buf, tid & 63);
        }
        if (g >= P0 - RA && (g - (P0 - RA)) % 8 == 0 && (g - (P0 - RA)) / 8 < 4) {
          const int r = (g - (P0 - RA)) / 8;
          ga.read_scale_pair(buf, ga_idx0, r, gsv);
          if (g > P0 - 1 && hit) gsv[2 * r] = gsv[2 * r + 1] = 1.f;
        }
        if (g == P0 - 1) {
          hit = ga_wave_hit(own, ga_hb_of(kt + 1));
          if (hit) {
            // (the empty asm keeps the reads inside this branch)
            asm volatile("" ::: "memory");
#pragma unroll
            for (int v = 0; v < 8; ++v)
              g_vec(a.v[v], ga.read_scale(buf, ga_idx0 + v),
                    ga.read_label(buf, ga_idx0 + v) - r0);
            gsv[0] = gsv[1] = 1.f;
          }
        }
        const int pc = g - P0;
        if (pc >= 0 && pc < 32) {
          const int v = pc >> 2, d = pc & 3;
          uint32_t& w = u4ref(a.v[v], d);
          w = g_dword_scale(w, gsv[v]);
        }
        if (g >= 2 * SL) {
          // (unconditional stores, as in mix_mainloop)
          const int q = g - 2 * SL;
#pragma unroll
          for (int u = (q * U + SL - 1) / SL; u < U && (u * SL) / U == q; ++u) {
            if (u < LB::U)
              b.store_unit_at(nx + BOFF, bo, u);
            else
              a.store_unit(nx, tid, u - LB::U);
          }
        }
      };
      hook_substep<FM, FN, SW>(acc, fa[0], fb[0], fa[1], fb[1], st, a_base, bb, xo[1],
                               [&](int q) __attribute__((always_inline)) { slot(q); });
      hook_substep<FM, FN, SW>(acc, fa[1], fb[1], fa[0], fb[0], st, a_base, bb, xo[2],
                               [&](int q) __attribute__((always_inline)) { slot(SL + q); });
      // B's units from one offset register that the empty asm makes opaque
      // each step, so their addresses are made where they are used instead
      // of held through the loop
      asm volatile("" : "+v"(bo));
      hook_substep<FM, FN, SW>(acc, fa[0], fb[0], fa[1], fb[1], st, a_base, bb, xo[3],
                               [&](int q) __attribute__((always_inline)) { slot(2 * SL + q); });
    } else {
      plain_substep<FM, FN, SW>(acc, fa[0], fb[0], fa[1], fb[1], st, a_base, bb, xo[1]);
      plain_substep<FM, FN, SW>(acc, fa[1], fb[1], fa[0], fb[0], st, a_base, bb, xo[2]);
      // (unconditional stores, as in mix_mainloop)
      store2_substep<FM, FN, SW>(acc, fa[0], fb[0], fa[1], fb[1], st, a_base, bb, xo[3], a, b,
                                 nx, nx + BOFF, tid, true);
    }
    __syncthreads();
    // the loads of k-step kt+3, spread over this substep
    const bool zero = kt + 3 == nk && nke != nk;
    if constexpr (GA) ga.issue(p, m0, k0 + kof(kt + 3), buf, zero, wave_u);
    a.prep_interior(p.A, p.lda, m0, k0 + kof(kt + 3), zero);
    b.prep_interior(p.B, p.ldb, n0, k0 + kof(kt + 3), zero);
    // (in the last k-step this reads a stale stage that is never used)
    load2_substep<FM, FN, SW>(acc, fa[1], fb[1], fa[0], fb[0], nx, a_base, bb, xo[0], a, b);
  };
  // two unconditional steps per iteration (see mix_mainloop)
  for (int kt = 0; kt < nke; kt += 2) {
    step(a1, b1, kt, 1);
    step(a0, b0, kt + 1, 0);
  }
  // the trailing loads must land before the registers are reused
  wait_dma();
}

// ----------------------------------------------------------------------
// The kernel.
// ----------------------------------------------------------------------
template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, int EPI>
__global__ void __launch_bounds__(kThreads, 1) gemm_kernel(GemmParams p) {
  constexpr int WM = BM / 2, WN = BN / 2;   // wave sub-tile
  constexpr int FM = WM / 32, FN = WN / 32; // 32x32 blocks per wave
  constexpr int SA = BM * kBK, SB = BN * kBK, STAGE = SA + SB;
  constexpr int RING = (BM + BN) * kRK * ring_stages<BM, BN>();
  constexpr bool SW = EPI == kEpiCE;  // transposed accumulators for row reductions
  constexpr bool Q8 = EPI == kEpiQ8Bf16 || EPI == kEpiQ8F32;  // e4m3fn operands made on load
  constexpr bool GA = EPI == kEpiGStoreBf16 || EPI == kEpiGStoreF32;  // CE gradient A on load
  // one K-contiguous operand, 256x256: the mixed loop (three D + two G panels)
  constexpr bool MIX = TGEMM_MIX && (A_KMAJOR != B_KMAJOR) && BM == 256 && BN == 256 && !Q8 && !GA;
  // neither operand K-contiguous, 256x256: two register sets per operand;
  // also a gradient A (either layout) with B contiguous along N
  constexpr bool REG2 = TGEMM_MIX && !B_KMAJOR && BM == 256 && BN == 256 && !Q8 &&
                        (GA || !A_KMAJOR);
  // (NT: the three-buffer loop for 256- and 192-row tiles, the ring for 128)
  constexpr int DMA3 = 2 * SA + 3 * SB;
  constexpr int NT_LDS = BM == 128 ? (RING > 2 * STAGE ? RING : 2 * STAGE)
                                   : (DMA3 > 2 * STAGE ? DMA3 : 2 * STAGE);
  constexpr int LDS_ELEMS =
      MIX ? DMA3 : ((A_KMAJOR && B_KMAJOR && !Q8 && !GA) ? NT_LDS : 2 * STAGE);
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
  // the gradient's staged scales and labels (two-set loop): one array per
  // register set, and the labels of K-contiguous gradient rows
  __shared__ __attribute__((aligned(16))) uint32_t gbuf0[REG2 && GA ? GaStage<A_KMAJOR>::kBufWords : 4];
  __shared__ __attribute__((aligned(16))) uint32_t gbuf1[REG2 && GA ? GaStage<A_KMAJOR>::kBufWords : 4];
  __shared__ __attribute__((aligned(16)))
  uint32_t glabs[REG2 && GA && A_KMAJOR ? GaStage<A_KMAJOR>::kLabWords : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, lc = lane & 31;

  // workgroup -> (tile, K chunk)
  int tile, ks;
  xcd_remap(blockIdx.x, p.tilesM * p.tilesN * p.splitk, p.splitk, tile, ks);
  int tm, tn;
  tile_coords(tile, p.tilesM, p.tilesN, p.groupM, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = ks * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  const bool aligned = p.aligned != 0;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS addressing of this lane's operand fragments (see read_frags).
  const int a_base = (wm * WM + lc) * kBK;
  const int b_base = SA + (wn * WN + lc) * kBK;
  int xo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) xo[s] = ((2 * s + h) ^ ((lc >> 1) & 7)) << 3;

  const bool interior = aligned && m0 + BM <= p.M && n0 + BN <= p.N && (kbeg % kBK) == 0 &&
                        ((kend - kbeg) % kBK) == 0 && p.lda < (1 << 23) && p.ldb < (1 << 23);
  bool staged = false;  // main loop done on a global->LDS copy path
  // (the direct copies move raw bf16, so Q8 operands take the register path)
  if constexpr (A_KMAJOR && B_KMAJOR && !Q8 && !GA) {
    if constexpr (BM != 128) {
      static_assert(2 * SA + 3 * SB <= LDS_ELEMS, "three B panels must fit");
      if (interior) {
        dma3_mainloop<BM, BN, FM, FN, SW>(p, m0, n0, kbeg, (kend - kbeg) / kBK, lds, wave, lane,
                                          a_base, b_base - SA, xo, acc);
        staged = true;
      }
    } else {
      if (interior) {
        ring_mainloop<BM, BN, FM, FN, A_KMAJOR, B_KMAJOR, SW>(p, m0, n0, kbeg,
                                                              (kend - kbeg) / kRK, lds, wave, lane,
                                                              wm, wn, acc);
        staged = true;
      }
    }
  }
  if constexpr (MIX) {
    if (interior) {
      mix_mainloop<BM, BN, FM, FN, A_KMAJOR, SW>(p, m0, n0, kbeg, (kend - kbeg) / kBK, lds,
                                                 lds + 3 * SA, tid, wave, lane, a_base,
                                                 b_base - SA, xo, acc);
      staged = true;
    }
  }
  if constexpr (REG2) {
    if (interior) {
      reg2_mainloop<BM, BN, FM, FN, SW, A_KMAJOR, GA>(p, m0, n0, kbeg, (kend - kbeg) / kBK, lds,
                                                      gbuf0, gbuf1, glabs, tid, a_base, b_base,
                                                      xo, acc);
      staged = true;
    }
  }
  // (both operands K-contiguous without the cast: interior tiles always take
  // a direct-copy loop above, so this path is not compiled for them)
  // (not compiled with the mixed or two-set loop: a third main loop merging
  // its accumulators into the epilogue makes the register allocator spill)
  constexpr bool kRegInterior = (!(A_KMAJOR && B_KMAJOR) || Q8 || GA) && !MIX && !REG2;
  if (kRegInterior && !staged && interior) {
    // Register path, interior tiles: one buffer load per 16-byte vector and
    // no bounds tests.  The loads of k-step kt+1 are issued right after the
    // barrier of k-step kt-1 (when the register set is free again), and the
    // set is written (transposed if needed) into the other LDS stage one
    // unit per matrix-core instruction during the third substep of kt.
    typename LoaderSel<A_KMAJOR, BM>::type la;
    typename LoaderSel<B_KMAJOR, BN>::type lb;
    using LA = typename LoaderSel<A_KMAJOR, BM>::type;
    const int nk = (kend - kbeg) / kBK;
    la.init_interior(p.lda, tid);
    lb.init_interior(p.ldb, tid);
    float qa = 0.f, qb = 0.f;
    if constexpr (Q8) {
      qa = p.qscales[0];
      qb = p.qscales[1];
    }
    la.load_interior(p.A, p.lda, m0, kbeg);
    lb.load_interior(p.B, p.ldb, n0, kbeg);
    if constexpr (GA) la.load_g(p, m0, kbeg, tid);
    if constexpr (Q8) {
      la.quantize(qa);
      lb.quantize(qb);
    }
    if constexpr (GA) {
#pragma unroll
      for (int u = 0; u < LA::L; ++u) la.rescale_one(u);
    }
    la.store(lds, tid);
    lb.store(lds + SA, tid);
    if (nk > 1) {
      la.load_interior(p.A, p.lda, m0, kbeg + kBK);
      lb.load_interior(p.B, p.ldb, n0, kbeg + kBK);
      if constexpr (GA) la.load_g(p, m0, kbeg + kBK, tid);
    }
    __syncthreads();
    bf16x8_t fa[2][FM], fb[2][FN];
    read_frags<FM, FN>(lds, a_base, b_base, xo[0], fa[0], fb[0]);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      const uint16_t* st = lds + cur * STAGE;
      uint16_t* nx = lds + (cur ^ 1) * STAGE;
      __builtin_amdgcn_sched_barrier(0);
      plain_substep<FM, FN, SW>(acc, fa[0], fb[0], fa[1], fb[1], st, a_base, b_base, xo[1]);
      if constexpr (Q8) {
        if (more) {
          la.quantize(qa);
          lb.quantize(qb);
        }
      }
      plain_substep<FM, FN, SW>(acc, fa[1], fb[1], fa[0], fb[0], st, a_base, b_base, xo[2]);
      // (GA: the next panel's gradient transform rides in this substep, just
      // before its stores; its scales and labels came with the panel)
      store2_substep<FM, FN, SW, GA>(acc, fa[0], fb[0], fa[1], fb[1], st, a_base, b_base, xo[3],
                                     la, lb, nx, nx + SA, tid, more);
      __syncthreads();
      if (kt + 2 < nk) {
        la.load_interior(p.A, p.lda, m0, kbeg + (kt + 2) * kBK);
        lb.load_interior(p.B, p.ldb, n0, kbeg + (kt + 2) * kBK);
        if constexpr (GA) la.load_g(p, m0, kbeg + (kt + 2) * kBK, tid);
      }
      // (in the last k-step this reads a stale stage that is never used)
      plain_substep<FM, FN, SW>(acc, fa[1], fb[1], fa[0], fb[0], nx, a_base, b_base, xo[0]);
    }
  } else if (!staged) {
    // General path: ragged edges, unaligned operands.  16-byte (or masked
    // element) loads into registers, one k-step ahead, then (transposing if
    // needed) stores into the other LDS stage.
    typename LoaderSel<A_KMAJOR, BM>::type la;
    typename LoaderSel<B_KMAJOR, BN>::type lb;
    using LA = typename LoaderSel<A_KMAJOR, BM>::type;
    const int nk = (kend - kbeg + kBK - 1) / kBK;
    la.load(p.A, p.lda, m0, p.M, kbeg, kend, aligned, tid);
    lb.load(p.B, p.ldb, n0, p.N, kbeg, kend, aligned, tid);
    if constexpr (GA) la.load_g(p, m0, kbeg, tid);
    float qa = 0.f, qb = 0.f;
    if constexpr (Q8) {
      qa = p.qscales[0];
      qb = p.qscales[1];
      la.quantize(qa);
      lb.quantize(qb);
    }
    if constexpr (GA) {
#pragma unroll
      for (int u = 0; u < LA::L; ++u) la.rescale_one(u);
    }
    la.store(lds, tid);
    lb.store(lds + SA, tid);
    __syncthreads();
    bf16x8_t fa[2][FM], fb[2][FN];
    read_frags<FM, FN>(lds, a_base, b_base, xo[0], fa[0], fb[0]);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        la.load(p.A, p.lda, m0, p.M, kbeg + (kt + 1) * kBK, kend, aligned, tid);
        lb.load(p.B, p.ldb, n0, p.N, kbeg + (kt + 1) * kBK, kend, aligned, tid);
        if constexpr (GA) la.load_g(p, m0, kbeg + (kt + 1) * kBK, tid);
      }
      const uint16_t* st = lds + cur * STAGE;
      uint16_t* nx = lds + (cur ^ 1) * STAGE;
      __builtin_amdgcn_sched_barrier(0);
      plain_substep<FM, FN, SW>(acc, fa[0], fb[0], fa[1], fb[1], st, a_base, b_base, xo[1]);
      plain_substep<FM, FN, SW>(acc, fa[1], fb[1], fa[0], fb[0], st, a_base, b_base, xo[2]);
      plain_substep<FM, FN, SW>(acc, fa[0], fb[0], fa[1], fb[1], st, a_base, b_base, xo[3]);
      if (more) {
        if constexpr (Q8) {
          la.quantize(qa);
          lb.quantize(qb);
        }
        if constexpr (GA) {
#pragma unroll
          for (int u = 0; u < LA::L; ++u) la.rescale_one(u);
        }
        la.store(nx, tid);
        lb.store(nx + SA, tid);
      }
      __syncthreads();
      // (in the last k-step this reads a stale stage that is never used)
      plain_substep<FM, FN, SW>(acc, fa[1], fb[1], fa[0], fb[0], nx, a_base, b_base, xo[0]);
    }
  }

  __syncthreads();  // every wave is done with LDS (the CE epilogue reuses it)
  // (split products always launch the fp32 store instance)
  if constexpr (EPI == kEpiStoreF32) {
    if (p.splitk > 1) {
      // K chunk ks of a split product: its fp32 partial goes to slice ks of
      // the workspace; a second kernel adds the slices in chunk order.
      GemmParams q = p;
      q.C = p.ws + (int64_t)ks * p.M * p.N;
      q.ldc = p.N;
      epilogue<kEpiStoreF32, FM, FN>(q, acc, m0, n0, wm * WM, wn * WN, 0, lane);
      return;
    }
  }
  epilogue<EPI, FM, FN, SW>(p, acc, m0, n0, wm * WM, wn * WN, tn * 2 + wn, lane);
}

// Host-side launch of one instantiation.
template <int BM, int BN, bool AK, bool BK>
hipError_t launch_gemm_tpl(int epi, const GemmParams& p, hipStream_t s) {
  const dim3 grid(p.tilesM * p.tilesN * p.splitk), block(kThreads);
  switch (epi) {
    case kEpiStoreBf16:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BK, kEpiStoreBf16>), grid, block, 0, s, p);
      break;
    case kEpiStoreF32:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BK, kEpiStoreF32>), grid, block, 0, s, p);
      break;
    case kEpiQ8Bf16:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BK, kEpiQ8Bf16>), grid, block, 0, s, p);
      break;
    case kEpiQ8F32:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BK, kEpiQ8F32>), grid, block, 0, s, p);
      break;
    case kEpiGStoreBf16:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BK, kEpiGStoreBf16>), grid, block, 0, s, p);
      break;
    case kEpiGStoreF32:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BK, kEpiGStoreF32>), grid, block, 0, s, p);
      break;
    case kEpiCE:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BK, kEpiCE>), grid, block, 0, s, p);
      break;
    default:  // (the OS epilogues belong to the fp8 kernel)
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 192x256 tiles: the NT store instances only (split products whose M is a
// multiple of 192; see choose_tile).
template <bool AK, bool BK>
hipError_t launch_gemm_192(int epi, const GemmParams& p, hipStream_t s) {
  if constexpr (AK && BK) {
    const dim3 grid(p.tilesM * p.tilesN * p.splitk), block(kThreads);
    if (epi == kEpiStoreBf16)
      hipLaunchKernelGGL((gemm_kernel<192, 256, true, true, kEpiStoreBf16>), grid, block, 0, s, p);
    else if (epi == kEpiStoreF32)
      hipLaunchKernelGGL((gemm_kernel<192, 256, true, true, kEpiStoreF32>), grid, block, 0, s, p);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  } else {
    (void)epi, (void)p, (void)s;
    return hipErrorInvalidValue;
  }
}

template <bool AK, bool BK>
hipError_t launch_gemm_layout(int cfg, int epi, const GemmParams& p, hipStream_t s) {
  if (cfg == kTile256) return launch_gemm_tpl<256, 256, AK, BK>(epi, p, s);
  if (cfg == kTile192) return launch_gemm_192<AK, BK>(epi, p, s);
  return launch_gemm_tpl<128, 128, AK, BK>(epi, p, s);
}

}  // namespace tgemm
