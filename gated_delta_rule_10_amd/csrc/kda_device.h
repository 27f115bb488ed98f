// kda_device.h -- device-side helpers shared by the libkda HIP kernels (gfx950).
//
// Matrix-core conventions used throughout (16x16 output tiles, wave64):
//   mma(acc, X, Y) accumulates acc[x][y] += sum_k X[x][k] * Y[y][k]; lane l
//   holds acc[4*(l/16) + i][l % 16] for i = 0..3 (the MFMA result layout).
//   X and Y fragments give lane l the 8 k-values of row (l % 16) that belong
//   to lane group g = l / 16.  Which 8 k-values a group holds is a free choice
//   as long as X and Y agree, because the products are summed over k.  Two
//   choices are used:
//     CK ("contiguous"):  k = k0 + 8g + {0..7}
//     SK ("split"):       k = k0 + 4g + {0..3}  and  k0 + 16 + 4g + {0..3}
//   SK matches the result layout: two result tiles covering k0..k0+15 and
//   k0+16..k0+31 (same y) packed together are an SK fragment, so a product's
//   result can feed the next product from registers without an LDS round trip.
//   bf16 fragments feed one V_MFMA_F32_16X16X32_BF16; fp32 fragments feed
//   eight V_MFMA_F32_16X16X4_F32 (element j of both fragments in instruction j).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Workgroup barrier for LDS hand-off.  On gfx950 it does not wait for
// outstanding global loads, so register prefetches stay in flight across it.
__device__ __forceinline__ void block_sync() { __syncthreads(); }

// exp2 on the hardware transcendental unit (inputs are pre-scaled by log2 e).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// K3's lower-bounded gate in log2 units ("How Kimi K3 Engineered Its Way to the
// Frontier", "How KDA updates its state"): for gate logit x of a channel with
// bias dt, log2(alpha) = s sigmoid(exp(A_log) (x + dt)) = s / (1 + 2^{-a (x + dt)}),
// where s = lower_bound log2(e) is folded on the host and a = exp(A_log) log2(e)
// (gate_head_factor).  Very large logits give s, very negative ones 0 (1 / inf).
__device__ __forceinline__ float gate_log2(float x, float a, float dt, float s) {
  return s * __builtin_amdgcn_rcpf(1.f + fast_exp2(-(a * (x + dt))));
}
__device__ __forceinline__ float gate_head_factor(float A_log) {
  return fast_exp2(A_log * kLog2e) * kLog2e;
}
// beta from a beta logit: 1 / (1 + e^{-x}).
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * kLog2e));
}

// ---------------------------------------------------------------- fragments
template <class OpT> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma(f32x4 &acc, const Frag<bf16> &x, const Frag<bf16> &y) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.v, y.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<float> &x, const Frag<float> &y) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.v[j], y.v[j], acc, 0, 0, 0);
}

// Load an SK fragment for row `row` of an LDS matrix (row stride `ld` elements).
__device__ __forceinline__ void lds_frag_sk(Frag<bf16> &f, const bf16 *base, int ld, int row,
                                            int k0, int g) {
  const bf16 *p = base + row * ld + k0 + 4 * g;
  const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p);
  const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p + 16);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void lds_frag_sk(Frag<float> &f, const float *base, int ld, int row,
                                            int k0, int g) {
  const float *p = base + row * ld + k0 + 4 * g;
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = a[i]; f.v[4 + i] = b[i]; }
}
// Load a CK fragment.
__device__ __forceinline__ void lds_frag_ck(Frag<bf16> &f, const bf16 *base, int ld, int row,
                                            int k0, int g) {
  f.v = *reinterpret_cast<const bf16x8 *>(base + row * ld + k0 + 8 * g);
}
__device__ __forceinline__ void lds_frag_ck(Frag<float> &f, const float *base, int ld, int row,
                                            int k0, int g) {
  const float *p = base + row * ld + k0 + 8 * g;
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = a[i]; f.v[4 + i] = b[i]; }
}
// Pack two result tiles (k-halves lo / hi of a 32-wide k step) into an SK fragment.
__device__ __forceinline__ void acc_frag_sk(Frag<bf16> &f, const f32x4 &lo, const f32x4 &hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = (bf16)lo[i]; f.v[4 + i] = (bf16)hi[i]; }
}
__device__ __forceinline__ void acc_frag_sk(Frag<float> &f, const f32x4 &lo, const f32x4 &hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = lo[i]; f.v[4 + i] = hi[i]; }
}

// ------------------------------------------- 16-wide k steps (k = 4g + {0..3})
// Four k-values per lane, the natural layout of V_MFMA_F32_16X16X16_BF16 and of
// a result tile's rows: a result tile acc[4g+i][y] is directly the Y fragment
// of rows y with k = 4g + i.
template <class OpT> struct Frag4;
template <> struct Frag4<bf16> { bf16x4 v; };
template <> struct Frag4<float> { f32x4 v; };

typedef short shortx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void mma16(f32x4 &acc, const Frag4<bf16> &x, const Frag4<bf16> &y) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, x.v),
                                                  __builtin_bit_cast(shortx4, y.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4 &acc, const Frag4<float> &x, const Frag4<float> &y) {
#pragma unroll
  for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.v[t], y.v[t], acc, 0, 0, 0);
}
__device__ __forceinline__ void lds_frag4(Frag4<bf16> &f, const bf16 *base, int ld, int row, int k0,
                                          int g) {
  f.v = *reinterpret_cast<const bf16x4 *>(base + row * ld + k0 + 4 * g);
}
__device__ __forceinline__ void lds_frag4(Frag4<float> &f, const float *base, int ld, int row,
                                          int k0, int g) {
  f.v = *reinterpret_cast<const f32x4 *>(base + row * ld + k0 + 4 * g);
}
__device__ __forceinline__ void acc_frag4(Frag4<bf16> &f, const f32x4 &a) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.v[i] = (bf16)a[i];
}
__device__ __forceinline__ void acc_frag4(Frag4<float> &f, const f32x4 &a) { f.v = a; }

// Register-only product of two 16x16 fp32 tiles held in the result layout
// (lane holds M[4g+i][l%16]): returns (B^T C) in the same layout, on fp32
// matrix cores.  Instruction i pairs row 4g+i of B and C across lane groups g.
__device__ __forceinline__ f32x4 rr_tn(const f32x4 &b, const f32x4 &c) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(b[i], c[i], acc, 0, 0, 0);
  return acc;
}

// ------------------------------------------------------- small vector I/O
// Buffer resource over `bytes` bytes starting at a wave-uniform address: memory
// instructions then take a scalar base plus a 32-bit per-lane offset, and any
// access at or past `bytes` reads zero / is dropped by the hardware range check.
// The base is made explicitly uniform so the descriptor lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t u = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  void *b = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}
constexpr int kNonTemporal = 2;  // streaming access: do not keep in the caches
// `off` is the per-lane byte offset, `soff` a wave-uniform byte offset (scalar).
__device__ __forceinline__ uint32_t buf_load_b32(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                 uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, kNonTemporal);
}
__device__ __forceinline__ f32x2 buf_load_f32x2(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                uint32_t soff = 0) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, kNonTemporal));
}
__device__ __forceinline__ u32x4 buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                               uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kNonTemporal);
}
__device__ __forceinline__ void buf_store_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, const f32x4 &v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kNonTemporal);
}
// The same through the caches (no streaming hint): partial lines written by
// different waves can merge in L2 before they reach memory.
__device__ __forceinline__ void buf_store_b128_cached(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                      const f32x4 &v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}

// Two consecutive elements of a row, widened to fp32.
__device__ __forceinline__ f32x2 load2(const bf16 *p) {
  const uint32_t u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
  f32x2 r;
  r[0] = __uint_as_float(u << 16);
  r[1] = __uint_as_float(u & 0xffff0000u);
  return r;
}
__device__ __forceinline__ f32x2 load2(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(p));
}

template <class T> __device__ __forceinline__ void store4(T *p, const f32x4 &v);
template <> __device__ __forceinline__ void store4<bf16>(bf16 *p, const f32x4 &v) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (bf16)v[i];
  *reinterpret_cast<bf16x4 *>(p) = r;
}
template <> __device__ __forceinline__ void store4<float>(float *p, const f32x4 &v) {
  *reinterpret_cast<f32x4 *>(p) = v;
}

template <class T> __device__ __forceinline__ void store2(T *p, float a, float b);
template <> __device__ __forceinline__ void store2<bf16>(bf16 *p, float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  *reinterpret_cast<bf16x2 *>(p) = v;
}
template <> __device__ __forceinline__ void store2<float>(float *p, float a, float b) {
  f32x2 v;
  v[0] = a;
  v[1] = b;
  *reinterpret_cast<f32x2 *>(p) = v;
}

}  // namespace kda
