// Device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core convention used everywhere (one 64-lane wavefront, 16x16 output):
//   A fragment (16 rows x 32 k): lane l holds A[l % 16][8*(l/16) + e], e = 0..7
//   B fragment (32 k x 16 cols): lane l holds B[8*(l/16) + e][l % 16]
//   C/D (16 x 16, fp32):         lane l holds C[4*(l/16) + j][l % 16],  j = 0..3
// bf16 and fp16 map to v_mfma_f32_16x16x32_{bf16,f16}.  fp32 runs the same
// fragment shape as eight v_mfma_f32_16x16x4_f32 steps, step p consuming
// element p of every lane, so k-slot (l/16) of step p is k = 8*(l/16) + p on
// both operands and the contraction covers all 32 k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
struct f32x8 { f32x4 lo, hi; };

template <typename T> struct FragOf;
template <> struct FragOf<bf16> { typedef bf16x8 type; };
template <> struct FragOf<f16> { typedef f16x8 type; };
template <> struct FragOf<float> { typedef f32x8 type; };

// Element type of the value-side products (P.V, V.G_h, V.y): fp32 stays fp32,
// 16-bit inputs run in fp16 (V converted exactly from bf16; P, G_h, y rounded
// to fp16's 11-bit significand).
template <typename T> struct ValueType { typedef f16 type; };
template <> struct ValueType<float> { typedef float type; };

__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f16x8 &a, const f16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8 &a, const f32x8 &b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], c, 0, 0, 0);
  return c;
}

// ---- scalar conversions ----------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }

// ---- fragment loads: 8 consecutive elements (16 B for 16-bit, 32 B for fp32) --
template <typename T> __device__ __forceinline__ typename FragOf<T>::type load8(const T *p);
template <> __device__ __forceinline__ bf16x8 load8<bf16>(const bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}
template <> __device__ __forceinline__ f16x8 load8<f16>(const f16 *p) {
  return *reinterpret_cast<const f16x8 *>(p);
}
template <> __device__ __forceinline__ f32x8 load8<float>(const float *p) {
  f32x8 r;
  r.lo = *reinterpret_cast<const f32x4 *>(p);
  r.hi = *reinterpret_cast<const f32x4 *>(p + 4);
  return r;
}

template <typename T> __device__ __forceinline__ typename FragOf<T>::type zero8();
template <> __device__ __forceinline__ bf16x8 zero8<bf16>() { return bf16x8{}; }
template <> __device__ __forceinline__ f16x8 zero8<f16>() { return f16x8{}; }
template <> __device__ __forceinline__ f32x8 zero8<float>() { return f32x8{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }

// Element e of a fragment, as fp32.
__device__ __forceinline__ float frag_elem(const bf16x8 &f, int e) { return (float)f[e]; }
__device__ __forceinline__ float frag_elem(const f16x8 &f, int e) { return (float)f[e]; }
__device__ __forceinline__ float frag_elem(const f32x8 &f, int e) { return e < 4 ? f.lo[e] : f.hi[e - 4]; }

// Build a fragment from 8 fp32 values.
template <typename T> __device__ __forceinline__ typename FragOf<T>::type pack8(const float *v);
template <> __device__ __forceinline__ bf16x8 pack8<bf16>(const float *v) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
  return r;
}
template <> __device__ __forceinline__ f16x8 pack8<f16>(const float *v) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (f16)v[e];
  return r;
}
template <> __device__ __forceinline__ f32x8 pack8<float>(const float *v) {
  return f32x8{f32x4{v[0], v[1], v[2], v[3]}, f32x4{v[4], v[5], v[6], v[7]}};
}

// Convert a fragment to another element type (bf16 -> fp16 is exact in range).
template <typename To, typename From>
__device__ __forceinline__ typename FragOf<To>::type convert8(const typename FragOf<From>::type &f) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = frag_elem(f, e);
  return pack8<To>(v);
}

// ---- 16-byte vector copies ---------------------------------------------------
struct alignas(16) U128 { uint32_t x, y, z, w; };

// A 16-byte chunk viewed as its elements.  A bit copy, not a pointer cast:
// type-based alias analysis may otherwise drop the write of the chunk that a
// read of its elements through another type depends on.
template <typename T> struct Elems16 { T e[16 / sizeof(T)]; };
template <typename T> __device__ __forceinline__ Elems16<T> elems16(const U128 &v) {
  return __builtin_bit_cast(Elems16<T>, v);
}
template <typename T> __device__ __forceinline__ U128 pack16(const Elems16<T> &v) {
  return __builtin_bit_cast(U128, v);
}

template <typename T> __device__ __forceinline__ uint32_t bits16(T x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, x);
}

// 16 bytes of Tin converted to Tout (8 x bf16 -> 8 x f16, or a plain copy
// when the types match).
template <typename Tin, typename Tout>
__device__ __forceinline__ U128 convert16(const U128 &v) {
  if constexpr (sizeof(Tin) == sizeof(Tout) && (sizeof(Tin) == 4 || __is_same(Tin, Tout))) {
    return v;
  } else if constexpr (__is_same(Tin, bf16) && __is_same(Tout, f16)) {
    // bf16 -> fp32 is a shift; fp32 -> fp16 of a bf16 value is exact in the
    // fp16 normal range, so the round-toward-zero pair conversion (one
    // instruction per two elements) gives the same bits there
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    U128 o;
    uint32_t *ow = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ow[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w[e] << 16),
                                                                      __uint_as_float(w[e] & 0xFFFF0000u)));
    return o;
  } else {
    const Elems16<Tin> ve = elems16<Tin>(v);
    U128 o;
    uint32_t *ow = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ow[e] = bits16(from_f32<Tout>(to_f32(ve.e[2 * e]))) |
              (bits16(from_f32<Tout>(to_f32(ve.e[2 * e + 1]))) << 16);
    return o;
  }
}

// ... and stored as one packed LDS write
template <typename Tin, typename Tout>
__device__ __forceinline__ void store_converted16(const U128 &v, Tout *dst) {
  *reinterpret_cast<U128 *>(dst) = convert16<Tin, Tout>(v);
}

// Eight fp16 values (one 16-byte chunk) as eight fp8 e5m2 bytes: e5m2 has
// fp16's sign and 5-bit exponent, so its byte is the fp16's upper byte (the
// mantissa rounded toward zero, subnormals included, and fp16's largest
// finite value maps to e5m2's, 57344).  v_perm_b32 picks bytes 1 and 3 of
// each of two words: one instruction per four elements.
__device__ __forceinline__ uint2 e5m2_of_f16x8(const U128 &h) {
  return make_uint2(__builtin_amdgcn_perm(h.y, h.x, 0x07050301u),
                    __builtin_amdgcn_perm(h.w, h.z, 0x07050301u));
}

// ---- raw buffer loads ----------------------------------------------------------
// A buffer resource covers [base, base + bytes); loads at byte offsets past
// `bytes` return zeros (the hardware range check), so ragged tails need no
// branches and the lane address is a 32-bit offset from a wave-uniform base.
// Word 3 = 0x00020000 is the raw (untyped, unswizzled) format of the gfx9
// family.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// The base and size must be wave-uniform; they are read from the first lane
// so the resource lives in scalar registers (a per-lane resource would make
// the compiler loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void *p = (void *)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}
__device__ __forceinline__ U128 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
  return U128{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0));
}
// A byte offset past every range: a load there reads zeros without a memory
// access, a store there is dropped.
constexpr uint32_t kNoLoad = 0xFFFFFFF0u;
// A store past the resource's range is dropped by the same check, so lanes
// that must not write pass kNoLoad instead of taking a branch.
__device__ __forceinline__ void buf_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)byte_off, 0, 0);
}
// A kernel's token range [t_begin, t_end) is covered by one resource built
// once; tile t0 is addressed with the lane offset plus (t0 - t_begin) * row
// bytes, and tiles past t_end read zeros without touching memory.  The range
// times the row size must stay below 2^32 bytes (hosts cap the range).
__device__ __forceinline__ uint32_t range_bytes(int t_begin, int t_end, uint32_t row_bytes) {
  return (uint32_t)max(t_end - t_begin, 0) * row_bytes;
}
// s_waitcnt vmcnt(0): every vector memory load issued so far has landed.
// Issued once after loop-invariant loads, it keeps the compiler from waiting
// on them (and so on the tile loads in flight) inside the tile loop.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Keep the instruction scheduler from moving code across this point (used to
// pin early LDS fragment reads ahead of the work that hides their latency).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// ---- wave reductions ---------------------------------------------------------
__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float wave_sum_xor(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

// Cross-lane sums without LDS traffic: the gfx950 permlane swaps exchange the
// upper 32 (16) lanes of one register with the lower 32 (16) lanes of
// another; swapping a value with itself and adding both results gives every
// lane v[l] + v[l ^ 32] (v[l] + v[l ^ 16]).
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// sum over the four 16-lane groups: lanes l, l^16, l^32, l^48
__device__ __forceinline__ float group4_sum(float v) { return sum_xor16(sum_xor32(v)); }
__device__ __forceinline__ float group4_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Sum over the 16 lanes of each DPP row (lanes 16r..16r+15); every lane of the
// row receives the total.  quad_perm [1,0,3,2] and [2,3,0,1] sum each quad,
// row_half_mirror pairs the two quads of each half-row, row_mirror the halves.
template <int CTRL> __device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}
// Inclusive prefix sum over the 64 lanes on the DPP network (every lane
// active): row_shr 1, 2, 4, 8 scan each 16-lane row, row_bcast 15 and 31
// carry the row totals into the rows above.
template <int CTRL> __device__ __forceinline__ int dpp_shr_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}
template <int CTRL, int ROWS> __device__ __forceinline__ int dpp_bcast_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_shr_i32<0x111>(x);
  x += dpp_shr_i32<0x112>(x);
  x += dpp_shr_i32<0x114>(x);
  x += dpp_shr_i32<0x118>(x);
  x += dpp_bcast_i32<0x142, 0xA>(x);
  x += dpp_bcast_i32<0x143, 0xC>(x);
  return x;
}

// v[l] + v[l ^ 8] within each 16-lane row (row_ror:8 pairs lane i with i +- 8)
__device__ __forceinline__ float sum_xor8(float v) { return v + dpp_f32<0x128>(v); }
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}
// sum / max over all 64 lanes, every lane receiving the result (all lanes active)
__device__ __forceinline__ float wave_sum_dpp(float v) { return group4_sum(row16_sum(v)); }
__device__ __forceinline__ float wave_max_dpp(float v) { return group4_max(row16_max(v)); }

// Fast hardware transcendentals (about 1 ulp).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// max(a, b) for non-NaN inputs (written as the median of a, b and +inf)
__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float hw_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }
__device__ __forceinline__ float hw_rsq(float x) { return __builtin_amdgcn_rsqf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace kvs
