// Device helpers shared by the libmuon kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16-byte register vector
typedef uint16_t bf16_t;   // bf16 stored as raw bits

constexpr int WAVE = 64;

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.  gfx950
// converts in hardware (v_cvt_pk_bf16_f32), branch-free.
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Load / store one element of a tensor whose dtype is a template parameter.
template <typename T> __device__ __forceinline__ float ld_as_f32(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld_as_f32<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld_as_f32<bf16_t>(const bf16_t* p, int64_t i) { return bf2f(p[i]); }

template <typename T> __device__ __forceinline__ void st_from_f32(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void st_from_f32<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st_from_f32<bf16_t>(bf16_t* p, int64_t i, float v) { p[i] = f2bf(v); }

// Value a stored element takes after rounding to T (identity for fp32).
template <typename T> __device__ __forceinline__ float round_to(float v);
template <> __device__ __forceinline__ float round_to<float>(float v) { return v; }
template <> __device__ __forceinline__ float round_to<bf16_t>(float v) { return bf2f(f2bf(v)); }

// Wave-wide sum with a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Row/column of accumulator register r of lane l in a 32x32 MFMA output block.
__device__ __forceinline__ int mfma32_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int mfma32_col(int lane) { return lane & 31; }

// Order a wave's LDS writes before its later reads of other lanes' data (and
// its reads before later overwrites), without a workgroup barrier.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// lr and wd of the update: from device memory when given (graph replays pick
// up new values), else the launch arguments.  Uniform loads.
__device__ __forceinline__ void update_scalars(const float* lrwd, float& lr, float& wd) {
  if (lrwd) {
    lr = lrwd[0];
    wd = lrwd[1];
  }
}

// 8 consecutive stored elements at a 16-byte aligned address, kept in their
// stored form (4 registers for bf16, 8 for fp32) until converted.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void to_f32(float* f) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) { f[2 * q] = __uint_as_float(v[q] << 16); f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u); }
  }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void to_f32(float* f) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) { f[q] = a[q]; f[q + 4] = b[q]; }
  }
};

// A pointer P such that P + b mn + e addresses element e of matrix b: the
// contiguous base itself, or matrix b's own address from the table moved
// back by b mn elements (on integers; only that matrix's elements are
// accessed through it).  b is uniform across the wave.
template <typename T>
__device__ __forceinline__ T* batch_view(T* contig, const void* const* tab, int64_t b, int64_t mn) {
  if (!tab) return contig;
  return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(tab[b]) - (uintptr_t)(b * mn) * sizeof(T));
}

// Start of stored row r of matrix b in a row table (R stored rows per
// matrix); b is uniform, r need not be.
template <typename T>
__device__ __forceinline__ T* row_of(const void* const* rows, int64_t b, int64_t R, int64_t r) {
  return reinterpret_cast<T*>(const_cast<void*>(rows[b * R + r]));
}

// Decoupled decay plus the orthogonal update on one element, fp32.
// W - lr (wd W + s O), its two fused multiply-adds spelled out so that every
// kernel rounds it the same way whatever the compiler would contract.
__device__ __forceinline__ float apply_update(float w, float o, float lr, float wd, float s) {
  return __builtin_fmaf(-lr, __builtin_fmaf(s, o, wd * w), w);
}

}  // namespace muon
