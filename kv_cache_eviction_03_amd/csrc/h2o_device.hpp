// Device-side helpers shared by the H2O kernels for gfx950: storage types,
// 16-byte chunk loads with conversion to fp32, wave reductions, MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

constexpr float kLog2e = 1.4426950408889634f;

// 2^x with the bare v_exp_f32 (about 1 ulp). The library exp2f wraps it in a
// rescale so that results below 2^-126 come out as denormals; softmax weights
// that small are irrelevant (they flush to 0 here), and the wrapper costs five
// extra VALU instructions per call.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Elements of T in one 16-byte chunk.
template <typename T> struct Chunk { static constexpr int N = 16 / sizeof(T); };

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// The same load marked nontemporal (streamed, not kept in the caches): data read once per
// kernel, such as a decode step's slot rows.
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Unpack a 16-byte chunk of T into fp32.
__device__ __forceinline__ void unpack(const uint4& v, float (&f)[4], float) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack(const uint4& v, float (&f)[8], _Float16) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
    f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
  }
}
__device__ __forceinline__ void unpack(const uint4& v, float (&f)[8], __bf16) {
  // bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename T>
__device__ __forceinline__ void load_f32(const T* p, float (&f)[Chunk<T>::N]) {
  unpack(ld16(p), f, T{});
}

// Butterfly reductions over groups of `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
  return ((uint64_t)hi << 32) | lo;
}
// DPP lane move of a float inside 16-lane rows (all lanes active).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
// DPP lane move of a 64-bit value inside 16-lane rows (all lanes active).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}
// Minimum over the wave, every lane gets it: four DPP steps inside each 16-lane row
// (symmetric pairings), then two shuffles across rows.
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  uint64_t w;
  w = dpp_u64<0xb1>(v); v = w < v ? w : v;     // quad_perm [1,0,3,2]
  w = dpp_u64<0x4e>(v); v = w < v ? w : v;     // quad_perm [2,3,0,1]
  w = dpp_u64<0x141>(v); v = w < v ? w : v;    // row_half_mirror
  w = dpp_u64<0x140>(v); v = w < v ? w : v;    // row_mirror
  w = shfl_xor_u64(v, 16); v = w < v ? w : v;
  w = shfl_xor_u64(v, 32); v = w < v ? w : v;
  return v;
}

// Wave-wide reductions whose result every lane receives as a uniform value: DPP steps
// inside each 16-lane row, then row_bcast15 / row_bcast31 fold the rows into lane 63,
// then readlane. The combination order is fixed, so the result is reproducible.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or(uint32_t old, uint32_t v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_fold_u32(uint32_t v, uint32_t identity, Op op) {
  v = op(v, dpp_or<0xb1, 0xf>(identity, v));     // quad_perm [1,0,3,2]
  v = op(v, dpp_or<0x4e, 0xf>(identity, v));     // quad_perm [2,3,0,1]
  v = op(v, dpp_or<0x141, 0xf>(identity, v));    // row_half_mirror
  v = op(v, dpp_or<0x140, 0xf>(identity, v));    // row_mirror: every lane has its row's value
  v = op(v, dpp_or<0x142, 0xa>(identity, v));    // row_bcast15 into rows 1 and 3
  v = op(v, dpp_or<0x143, 0xc>(identity, v));    // row_bcast31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ float wave_max_uniform(float v) {
  return __uint_as_float(wave_fold_u32(__float_as_uint(v), __float_as_uint(-INFINITY),
      [](uint32_t a, uint32_t b) { return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b))); }));
}
__device__ __forceinline__ float wave_sum_uniform(float v) {
  return __uint_as_float(wave_fold_u32(__float_as_uint(v), 0u,
      [](uint32_t a, uint32_t b) { return __float_as_uint(__uint_as_float(a) + __uint_as_float(b)); }));
}
__device__ __forceinline__ uint32_t wave_min_u32_uniform(uint32_t v) {
  return wave_fold_u32(v, ~0u, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
// Minimum of 64-bit keys over the wave as two 32-bit folds (high word, then the low word
// among lanes holding that high word).
__device__ __forceinline__ uint64_t wave_min_u64_uniform(uint64_t v) {
  const uint32_t hi = wave_min_u32_uniform((uint32_t)(v >> 32));
  const uint32_t lo = wave_min_u32_uniform((uint32_t)(v >> 32) == hi ? (uint32_t)v : ~0u);
  return ((uint64_t)hi << 32) | lo;
}

// 16x16x32 MFMA, fp32 accumulate (gfx950). Lane l supplies A[l%16][k-group l/16]
// and B[k-group l/16][l%16]; D[4*(l/16)+i][l%16] comes back in element i.
__device__ __forceinline__ f32x4 mfma16x16x32(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- OCP FP8 E4M3 slot codes (one byte per element: sign, 4 exponent bits with bias 7,
// 3 mantissa bits; largest finite value 448). gfx950's conversions use this format.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
// Nontemporal 8-byte load (E4M3 slot rows: read once per step, like ld16_nt).
__device__ __forceinline__ uint2 ld8_nt(const void* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(x[0], x[1]);
}
__device__ __forceinline__ void st8(void* p, const uint2& v) { *reinterpret_cast<uint2*>(p) = v; }

// One 16-byte chunk of T (8 elements) -> its 8 codes: each element times `inv` (one fp32
// rounding), clamped to +-448, then the hardware's round-to-nearest-even conversion.
// Element i goes to byte i.
template <typename T>
__device__ __forceinline__ uint2 quant_e4m3(const uint4& x, float inv) {
  float f[8];
  unpack(x, f, T{});
  uint32_t w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = __builtin_amdgcn_fmed3f(f[4 * i + e] * inv, -448.f, 448.f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], r, true);
    w[i] = (uint32_t)r;
  }
  return make_uint2(w[0], w[1]);
}

// 8 codes -> fp32 (exact: every E4M3 value is an fp32 value).
template <typename T>
__device__ __forceinline__ void unpack(const uint2& v, float (&f)[8], T) {
  const uint32_t w[2] = {v.x, v.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    f[4 * i] = lo.x; f[4 * i + 1] = lo.y; f[4 * i + 2] = hi.x; f[4 * i + 3] = hi.y;
  }
}

// Slot storage: a lane's share of a slot row is one 16-byte chunk of T, or, with E4M3
// slots (F8), the 8 codes of the same elements.
template <typename T, bool F8> struct SlotChunk {
  typedef uint4 type;
  typedef T elem;
  __device__ static type load(const elem* p) { return ld16(p); }
  __device__ static void store(elem* p, const type& v) { st16(p, v); }
};
template <typename T> struct SlotChunk<T, true> {
  static_assert(sizeof(T) == 2, "E4M3 slots take fp16 or bf16 inputs");
  typedef uint2 type;
  typedef uint8_t elem;
  // Slot rows are loaded nontemporal, as the 16-bit decode kernels load theirs: a step
  // reads each once, and a deep model visits every other layer before it comes back.
  __device__ static type load(const elem* p) { return ld8_nt(p); }
  __device__ static void store(elem* p, const type& v) { st8(p, v); }
};

template <typename T> struct Vec8;
template <> struct Vec8<_Float16> { typedef f16x8 type; typedef f16x4 half; };
template <> struct Vec8<__bf16> { typedef bf16x8 type; typedef bf16x4 half; };

}  // namespace h2o
