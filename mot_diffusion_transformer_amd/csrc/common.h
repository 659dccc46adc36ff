// Device-side helpers shared by the HIP kernels of the MoT world-action-model
// forward pass: element types, bf16 conversion, wavefront reductions and the
// GEMM epilogues.  gfx950 only (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 bits in memory

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

#define WAM_DEV __device__ __forceinline__

// ---------------------------------------------------------------- element conversion
template <class T> WAM_DEV float to_f32(T v);
template <> WAM_DEV float to_f32<float>(float v) { return v; }
template <> WAM_DEV float to_f32<bf16_t>(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

template <class T> WAM_DEV T from_f32(float f);
template <> WAM_DEV float from_f32<float>(float f) { return f; }
// Round to nearest, ties to even (the IEEE conversion the compiler emits).
template <> WAM_DEV bf16_t from_f32<bf16_t>(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

WAM_DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
WAM_DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
WAM_DEV uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)from_f32<bf16_t>(lo) | ((uint32_t)from_f32<bf16_t>(hi) << 16);
}

// ---------------------------------------------------------------- wavefront reductions
WAM_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
WAM_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

WAM_DEV float silu_f(float z) { return z / (1.0f + __expf(-z)); }
WAM_DEV float gelu_f(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// ---------------------------------------------------------------- GEMM epilogues
// Every GEMM computes acc[m][n] = sum_k A[m][k] W[n][k] (fp32 accumulation)
// and hands each finished element to exactly one epilogue call, so results
// never depend on scheduling.

// out[m][n] = act(acc + bias[n]) in float32 (act: 0 none, 1 SiLU).
template <class T>
struct EpiF32 {
  float* out;
  int ldo;
  const T* bias;
  int act;
  WAM_DEV void operator()(int m, int n, float acc) const {
    float v = acc + (bias ? to_f32<T>(bias[n]) : 0.0f);
    if (act == 1) v = silu_f(v);
    out[(size_t)m * ldo + n] = v;
  }
};

// Merged q|k|v projection, scattered head-major: column n of the 3*H*dh
// outputs is (which = n / (H dh), head, e); row m is (sample b, token t).
// Destination [b][head][t][e] of the q, k or v base.
template <class T>
struct EpiQKV {
  T* q;
  T* k;
  T* v;
  const T* bias;
  int tokens;  // tokens per sample
  int H, dh;
  WAM_DEV void operator()(int m, int n, float acc) const {
    const int D = H * dh;
    int which = n / D, r = n - which * D;
    int h = r / dh, e = r - h * dh;
    int b = m / tokens, t = m - b * tokens;
    T* base = which == 0 ? q : (which == 1 ? k : v);
    base[(((size_t)b * H + h) * tokens + t) * dh + e] = from_f32<T>(acc + to_f32<T>(bias[n]));
  }
};

// Gated residual: x[m][n] += gate[n] * (acc + bias[n]), x float32.
template <class T>
struct EpiGateRes {
  float* x;
  int ldx;
  const float* gate;
  const T* bias;
  WAM_DEV void operator()(int m, int n, float acc) const {
    float* p = x + (size_t)m * ldx + n;
    *p = *p + gate[n] * (acc + to_f32<T>(bias[n]));
  }
};

// out[m][n] = GELU(acc + bias[n]) in the model dtype.
template <class T>
struct EpiGelu {
  T* out;
  int ldo;
  const T* bias;
  WAM_DEV void operator()(int m, int n, float acc) const {
    out[(size_t)m * ldo + n] = from_f32<T>(gelu_f(acc + to_f32<T>(bias[n])));
  }
};
