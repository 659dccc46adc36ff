// Device-side helpers shared by the HIP kernels of the MoT world-action-model
// forward pass: element types, bf16 conversion, wavefront reductions and the
// GEMM epilogues.  gfx950 only (64-lane wavefronts).
#pragma once

#include <utility>
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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats to packed bf16 (lo in the low half), round to nearest even: one v_cvt_pk_bf16_f32
WAM_DEV uint32_t pack_bf2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// f(std::integral_constant<int, 0>{}), ..., f(...<int, N-1>{}): a loop body
// expanded at compile time, so indices into register arrays stay constants
template <class F, int... Is>
WAM_DEV void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
WAM_DEV void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------- direct loads into LDS
#define WAM_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Buffer descriptor over `bytes` bytes at p (raw, stride 0; reads past the
// end return zero) and the 16-byte-per-lane buffer load straight into LDS:
// lane l's 16 bytes land at lds + 16 l.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
WAM_DEV BufRsrc buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
}
WAM_DEV void buf_load_lds16(BufRsrc r, void* lds, uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, WAM_LDS_PTR(lds), 16, voffset, soffset, 0, 0);
}
// ---------------------------------------------------------------- wavefront reductions
WAM_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over a wavefront, returned in every lane: DPP adds inside each 16-lane
// row (pairs, quads, half rows, rows), then the four row sums in row order.
// (A shuffle butterfly is six LDS-crossbar round trips, each waited for.)
WAM_DEV float wave_sum_dpp(float x) {
  auto dpp = [](float v, int ctrl_id) {
    const int u = __builtin_bit_cast(int, v);
    int r;
    switch (ctrl_id) {
      case 0: r = __builtin_amdgcn_update_dpp(0, u, 0xB1, 0xF, 0xF, true); break;  // quad_perm [1,0,3,2]
      case 1: r = __builtin_amdgcn_update_dpp(0, u, 0x4E, 0xF, 0xF, true); break;  // quad_perm [2,3,0,1]
      case 2: r = __builtin_amdgcn_update_dpp(0, u, 0x141, 0xF, 0xF, true); break;  // row_half_mirror
      default: r = __builtin_amdgcn_update_dpp(0, u, 0x140, 0xF, 0xF, true); break;  // row_mirror
    }
    return __builtin_bit_cast(float, r);
  };
  x += dpp(x, 0);
  x += dpp(x, 1);
  x += dpp(x, 2);
  x += dpp(x, 3);
  const int u = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 48));
  return (r0 + r1) + (r2 + r3);
}

// The value of lane l combined with that of lane l ^ 32, on the VALU
// (v_permlane32_swap exchanges the two halves of the wavefront; a shuffle
// would go through LDS, a round trip on the critical path).  Max and the
// two-operand sum are commutative, so the result equals v op shfl_xor(v, 32)
// to the bit.
WAM_DEV float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
WAM_DEV float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
WAM_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

WAM_DEV float silu_f(float z) { return z / (1.0f + __expf(-z)); }
// GELU(z) = z Phi(z) with Phi(z) = (1 + erf(z / sqrt 2)) / 2 (the exact-erf
// form).  erf comes from Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (|error| <= 1.5e-7, far below bf16 resolution):
// for x >= 0, erf(x) = 1 - q(t) exp(-x^2), q(t) = a1 t + ... + a5 t^5,
// t = 1 / (1 + p x).  Phi of a negative argument is taken as q e / 2
// directly, so no 1 - (nearly 1) cancellation occurs.
WAM_DEV float gelu_f(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float q = fmaf(1.061405429f, t, -1.453152027f);
  q = fmaf(q, t, 1.421413741f);
  q = fmaf(q, t, -0.284496736f);
  q = fmaf(q, t, 0.254829592f);
  q *= t;
  const float half_tail = 0.5f * q * __builtin_amdgcn_exp2f(-1.4426950408889634f * x * x);  // (1 - erf(x)) / 2
  return z * (z >= 0.0f ? 1.0f - half_tail : half_tail);
}

// ---------------------------------------------------------------- GEMM epilogues
// Every GEMM computes acc[m][n] = sum_k A[m][k] W[n][k] (fp32 accumulation)
// and hands each finished element to exactly one epilogue call, so results
// never depend on scheduling.  operator() takes one element; store4() takes
// four consecutive columns n..n+3 (n % 4 == 0, n + 3 < N) of one row, and
// is pre4() (the loads of everything the four outputs need: bias, gate,
// residual) followed by fin4() (the arithmetic and the store).  A caller
// with several groups to store calls every pre4() before the first fin4():
// the compiler must assume a store may alias a later load, so loads
// interleaved with stores wait one memory round trip each.
// (Raw bits: converting right after the load, bf16 to float, would make the
// compiler wait for that load there.)
struct Pre4 {
  uint4 a, b, c;
};

template <class T> struct Vec4Ld;
template <> struct Vec4Ld<float> {
  WAM_DEV static float4 ld(const float* p) { return *(const float4*)p; }
  WAM_DEV static void st(float* p, float4 v) { *(float4*)p = v; }
};
template <> struct Vec4Ld<bf16_t> {
  WAM_DEV static float4 ld(const bf16_t* p) {
    uint2 u = *(const uint2*)p;
    return make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
  }
  WAM_DEV static void st(bf16_t* p, float4 v) {
    uint2 u;
    u.x = pack_bf2(v.x, v.y);
    u.y = pack_bf2(v.z, v.w);
    *(uint2*)p = u;
  }
};

WAM_DEV float4 add4(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }

// Four consecutive values as raw bits (uint4; bf16 in .x, .y) and back to float.
template <class T> struct Raw4;
template <> struct Raw4<float> {
  WAM_DEV static uint4 ld(const float* p) { return *(const uint4*)p; }
  WAM_DEV static float4 f(uint4 u) { return __builtin_bit_cast(float4, u); }
  WAM_DEV static uint32_t ld1(const float* p) { return __builtin_bit_cast(uint32_t, *p); }
  WAM_DEV static float f1(uint32_t u) { return __builtin_bit_cast(float, u); }
};
template <> struct Raw4<bf16_t> {
  WAM_DEV static uint4 ld(const bf16_t* p) {
    const uint2 u = *(const uint2*)p;
    return make_uint4(u.x, u.y, 0u, 0u);
  }
  WAM_DEV static float4 f(uint4 u) { return make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y)); }
  WAM_DEV static uint32_t ld1(const bf16_t* p) { return (uint32_t)*(const unsigned short*)p; }
  WAM_DEV static float f1(uint32_t u) { return bf_lo(u); }
};

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
  WAM_DEV Pre4 pre4(int, int n) const {
    Pre4 p;
    p.a = bias ? Raw4<T>::ld(bias + n) : make_uint4(0u, 0u, 0u, 0u);
    return p;
  }
  WAM_DEV void fin4(int m, int n, float4 v, const Pre4& p) const {
    v = add4(v, Raw4<T>::f(p.a));
    if (act == 1) v = make_float4(silu_f(v.x), silu_f(v.y), silu_f(v.z), silu_f(v.w));
    *(float4*)(out + (size_t)m * ldo + n) = v;
  }
  WAM_DEV void store4(int m, int n, float4 v) const { fin4(m, n, v, pre4(m, n)); }
};

// n / d for a divisor d >= 1 fixed at launch, exact for 0 <= n < 2^31, in a
// multiply-high, an add and a shift (a full 32-bit division is a few dozen
// instructions): the round-up method of Granlund and Montgomery ("Division
// by invariant integers using multiplication", 1994) with l = ceil(log2 d)
// and the multiplier 2^32 + m = floor(2^(32+l) / d) + 1, so that
// n / d = (n + mulhi(n, m)) >> l; below 2^31 the sum fits in 32 bits.
struct FastDiv {
  uint32_t m = 1, l = 0;  // d = 1
  WAM_DEV int div(int n) const { return (int)(((uint32_t)n + __umulhi((uint32_t)n, m)) >> l); }
};
static inline FastDiv fast_div(int d) {
  FastDiv f;
  uint32_t l = 0;
  while ((1ull << l) < (unsigned long long)d) ++l;
  f.l = l;
  f.m = (uint32_t)((1ull << (32 + l)) / (unsigned long long)d + 1 - (1ull << 32));
  return f;
}

// Merged q|k|v projection, scattered head-major: column n of the 3*H*dh
// outputs is (which = n / (H dh), head, e); row m is (sample b, token t).
// q and k go to [b][head][t][e]; v goes TRANSPOSED to [b][head][e][t], the
// layout the attention's P.V product reads (keys contiguous).
template <class T>
struct EpiQKV {
  T* q;
  T* k;
  T* v;
  const T* bias;
  int tokens;  // tokens per sample
  int H, dh;
  FastDiv div_D, div_dh, div_tok;  // by H * dh, dh, tokens (fast_div, set by launch_qkv)
  WAM_DEV T* dst(int m, int n) const {
    const int D = H * dh;
    const int which = div_D.div(n), r = n - which * D;
    const int h = div_dh.div(r), e = r - h * dh;
    const int b = div_tok.div(m), t = m - b * tokens;
    if (which == 2) return v + (((size_t)b * H + h) * dh + e) * tokens + t;
    return (which == 0 ? q : k) + (((size_t)b * H + h) * tokens + t) * dh + e;
  }
  WAM_DEV void operator()(int m, int n, float acc) const {
    *dst(m, n) = from_f32<T>(acc + to_f32<T>(bias[n]));
  }
  WAM_DEV bool q_or_k_columns(int n_lo, int n_hi) const { return n_hi <= 2 * H * dh; }
  // four consecutive columns of one row (q or k; dh % 4 == 0 keeps them in one head)
  WAM_DEV Pre4 pre4(int, int n) const {
    Pre4 p;
    p.a = Raw4<T>::ld(bias + n);
    return p;
  }
  WAM_DEV void fin4(int m, int n, float4 a, const Pre4& p) const { Vec4Ld<T>::st(dst(m, n), add4(a, Raw4<T>::f(p.a))); }
  WAM_DEV void store4(int m, int n, float4 a) const { fin4(m, n, a, pre4(m, n)); }
  // eight consecutive q or k columns of a bf16 output (dh % 8 == 0 keeps them
  // in one head): one 16-byte store
  WAM_DEV uint4 pre8(int, int n) const { return *(const uint4*)(bias + n); }
  WAM_DEV void fin8(int m, int n, float4 lo, float4 hi, uint4 b) const {
    *(uint4*)dst(m, n) = make_uint4(pack_bf2(lo.x + bf_lo(b.x), lo.y + bf_hi(b.x)), pack_bf2(lo.z + bf_lo(b.y), lo.w + bf_hi(b.y)),
                                    pack_bf2(hi.x + bf_lo(b.z), hi.y + bf_hi(b.z)), pack_bf2(hi.z + bf_lo(b.w), hi.w + bf_hi(b.w)));
  }
  // value columns only, with whole groups of four tokens per sample: four
  // consecutive rows (tokens) of one value column are contiguous in V^T
  WAM_DEV bool v_columns(int n_lo) const { return n_lo >= 2 * H * dh && tokens % 4 == 0; }
  // rows m..m+3 (m % 4 == 0) of value column n: one 8-byte store along V^T
  // (head * dh + e is n - 2 D itself, so only the sample needs a division)
  WAM_DEV Pre4 preT4(int, int n) const {
    Pre4 p;
    p.a.x = Raw4<T>::ld1(bias + n);
    return p;
  }
  WAM_DEV void finT4(int m, int n, float4 a, const Pre4& pr) const {
    const int D = H * dh, b = div_tok.div(m), t = m - b * tokens;
    T* p = v + ((size_t)b * D + (n - 2 * D)) * tokens + t;
    const float c = Raw4<T>::f1(pr.a.x);
    Vec4Ld<T>::st(p, make_float4(a.x + c, a.y + c, a.z + c, a.w + c));
  }
  WAM_DEV void storeT4(int m, int n, float4 a) const { finT4(m, n, a, preT4(m, n)); }
};

// Transposed value projection computed directly: the GEMM runs with the
// value rows of W_qkv as A (row r = head*dh + e) and the normalised tokens
// as the second operand (column n = b*tokens + t), so acc[r][n] = v[n][r]
// and the natural row-major result is V^T [b][head][e][t] -- tokens stay
// contiguous and the stores coalesce.
template <class T>
struct EpiVT {
  T* v;
  const T* bias;  // the value third of b_qkv, indexed by r
  int tokens, D;
  FastDiv div_tok;  // by tokens
  WAM_DEV T* dst(int r, int n) const {
    const int b = div_tok.div(n), t = n - b * tokens;
    return v + ((size_t)b * D + r) * tokens + t;
  }
  WAM_DEV void operator()(int r, int n, float acc) const { *dst(r, n) = from_f32<T>(acc + to_f32<T>(bias[r])); }
  // n..n+3 stay in one sample when tokens % 4 == 0 (checked through epi_rows_ok)
  WAM_DEV Pre4 pre4(int r, int) const {
    Pre4 p;
    p.a.x = Raw4<T>::ld1(bias + r);
    return p;
  }
  WAM_DEV void fin4(int r, int n, float4 a, const Pre4& p) const {
    const float b = Raw4<T>::f1(p.a.x);
    Vec4Ld<T>::st(dst(r, n), make_float4(a.x + b, a.y + b, a.z + b, a.w + b));
  }
  WAM_DEV void store4(int r, int n, float4 a) const { fin4(r, n, a, pre4(r, n)); }
};

// The q|k|v projection of selected rows of one sample (selective reuse):
// q stays compact, [head][m][e] for the M rows; k and v (transposed) of row
// m go to token tok[m] of a cache of `tokens` tokens.
template <class T>
struct EpiQKVMap {
  T* q;
  T* k;
  T* v;
  const T* bias;
  int rows;
  int H, dh;
  const int* tok;
  int tokens;
  FastDiv div_D, div_dh;  // by H * dh, dh
  WAM_DEV T* dst(int m, int n) const {
    const int D = H * dh;
    const int which = div_D.div(n), r = n - which * D;
    const int h = div_dh.div(r), e = r - h * dh;
    if (which == 0) return q + ((size_t)h * rows + m) * dh + e;
    if (which == 1) return k + ((size_t)h * tokens + tok[m]) * dh + e;
    return v + ((size_t)h * dh + e) * tokens + tok[m];
  }
  WAM_DEV void operator()(int m, int n, float acc) const { *dst(m, n) = from_f32<T>(acc + to_f32<T>(bias[n])); }
  WAM_DEV bool q_or_k_columns(int n_lo, int n_hi) const { return n_hi <= 2 * H * dh; }
  WAM_DEV Pre4 pre4(int, int n) const {
    Pre4 p;
    p.a = Raw4<T>::ld(bias + n);
    return p;
  }
  WAM_DEV void fin4(int m, int n, float4 a, const Pre4& p) const { Vec4Ld<T>::st(dst(m, n), add4(a, Raw4<T>::f(p.a))); }
  WAM_DEV void store4(int m, int n, float4 a) const { fin4(m, n, a, pre4(m, n)); }
};

// V^T of selected rows (the swapped GEMM): column n goes to token tok[n].
template <class T>
struct EpiVTMap {
  T* v;
  const T* bias;  // the value third of b_qkv, indexed by r
  int tokens;
  const int* tok;
  WAM_DEV void operator()(int r, int n, float acc) const {
    v[(size_t)r * tokens + tok[n]] = from_f32<T>(acc + to_f32<T>(bias[r]));
  }
  // not reached: the columns are not contiguous (epi_rows_ok is false)
  WAM_DEV Pre4 pre4(int, int) const { return Pre4{}; }
  WAM_DEV void fin4(int r, int n, float4 a, const Pre4&) const {
    (*this)(r, n, a.x);
    (*this)(r, n + 1, a.y);
    (*this)(r, n + 2, a.z);
    (*this)(r, n + 3, a.w);
  }
  WAM_DEV void store4(int r, int n, float4 a) const { fin4(r, n, a, Pre4{}); }
};

// Whether four consecutive columns n..n+3 of a row may go through store4:
// not for the value columns of EpiQKV (transposed, so not contiguous), and
// for EpiVT only when the four columns stay within one sample.
template <class E>
WAM_DEV bool epi_rows_ok(const E&, int, int) { return true; }
template <class T>
WAM_DEV bool epi_rows_ok(const EpiQKV<T>& e, int lo, int hi) { return e.q_or_k_columns(lo, hi); }
template <class T>
WAM_DEV bool epi_rows_ok(const EpiVT<T>& e, int, int) { return (e.tokens % 4) == 0; }
template <class T>
WAM_DEV bool epi_rows_ok(const EpiQKVMap<T>& e, int lo, int hi) { return e.q_or_k_columns(lo, hi); }
template <class T>
WAM_DEV bool epi_rows_ok(const EpiVTMap<T>&, int, int) { return false; }
// Column path of the tiled epilogue (storeT4: four consecutive rows of one
// column); only the value columns of the q|k|v projection have it.
template <class E>
WAM_DEV bool epi_cols_ok(const E&, int) { return false; }
template <class T>
WAM_DEV bool epi_cols_ok(const EpiQKV<T>& e, int lo) { return e.v_columns(lo); }
template <class E>
WAM_DEV void epi_storeT4(const E&, int, int, float4) {}
template <class T>
WAM_DEV void epi_storeT4(const EpiQKV<T>& e, int m, int n, float4 a) { e.storeT4(m, n, a); }
template <class E>
WAM_DEV Pre4 epi_preT4(const E&, int, int) { return Pre4{}; }
template <class T>
WAM_DEV Pre4 epi_preT4(const EpiQKV<T>& e, int m, int n) { return e.preT4(m, n); }
template <class E>
WAM_DEV void epi_finT4(const E&, int, int, float4, const Pre4&) {}
template <class T>
WAM_DEV void epi_finT4(const EpiQKV<T>& e, int m, int n, float4 a, const Pre4& p) { e.finT4(m, n, a, p); }

// Raw float32 accumulators of one K split: part[m][n] of the tile row-major
// [M][N]; split s writes at part + s * split_stride (epi_split).
struct EpiPart {
  float* part;
  int N;
  size_t split_stride;
  WAM_DEV void operator()(int m, int n, float a) const { part[(size_t)m * N + n] = a; }
  WAM_DEV Pre4 pre4(int, int) const { return Pre4{}; }
  WAM_DEV void fin4(int m, int n, float4 a, const Pre4&) const { *(float4*)(part + (size_t)m * N + n) = a; }
  WAM_DEV void store4(int m, int n, float4 a) const { fin4(m, n, a, Pre4{}); }
};
// Selects the output of K split s (a no-op for every final epilogue).
template <class E>
WAM_DEV void epi_split(E&, int) {}
WAM_DEV void epi_split(EpiPart& e, int s) { e.part += (size_t)s * e.split_stride; }

// Gated residual: x[m][n] += gate[n] * (acc + bias[n]), x float32.  With
// gate_stride != 0 the gate is per sample: rows m of group m / rows_per_group
// use gate + group * gate_stride.
template <class T>
struct EpiGateRes {
  float* x;
  int ldx;
  const float* gate;
  const T* bias;
  int rows_per_group = 1;
  size_t gate_stride = 0;
  WAM_DEV const float* g_row(int m) const {
    return gate_stride ? gate + (size_t)(m / rows_per_group) * gate_stride : gate;
  }
  WAM_DEV void operator()(int m, int n, float acc) const {
    float* p = x + (size_t)m * ldx + n;
    *p = *p + g_row(m)[n] * (acc + to_f32<T>(bias[n]));
  }
  WAM_DEV Pre4 pre4(int m, int n) const {
    Pre4 p;
    p.a = Raw4<float>::ld(x + (size_t)m * ldx + n);  // the residual
    p.b = Raw4<float>::ld(g_row(m) + n);
    p.c = Raw4<T>::ld(bias + n);
    return p;
  }
  WAM_DEV void fin4(int m, int n, float4 a, const Pre4& p) const {
    const float4 xv = Raw4<float>::f(p.a), g = Raw4<float>::f(p.b), b = Raw4<T>::f(p.c);
    *(float4*)(x + (size_t)m * ldx + n) = make_float4(xv.x + g.x * (a.x + b.x), xv.y + g.y * (a.y + b.y),
                                                      xv.z + g.z * (a.z + b.z), xv.w + g.w * (a.w + b.w));
  }
  WAM_DEV void store4(int m, int n, float4 a) const { fin4(m, n, a, pre4(m, n)); }
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
  WAM_DEV Pre4 pre4(int, int n) const {
    Pre4 p;
    p.a = Raw4<T>::ld(bias + n);
    return p;
  }
  WAM_DEV void fin4(int m, int n, float4 a, const Pre4& p) const {
    const float4 v = add4(a, Raw4<T>::f(p.a));
    Vec4Ld<T>::st(out + (size_t)m * ldo + n, make_float4(gelu_f(v.x), gelu_f(v.y), gelu_f(v.z), gelu_f(v.w)));
  }
  WAM_DEV void store4(int m, int n, float4 a) const { fin4(m, n, a, pre4(m, n)); }
  // eight consecutive columns of a bf16 output: one 16-byte store
  WAM_DEV uint4 pre8(int, int n) const { return *(const uint4*)(bias + n); }
  WAM_DEV void fin8(int m, int n, float4 lo, float4 hi, uint4 b) const {
    *(uint4*)(out + (size_t)m * ldo + n) = gelu8(lo, hi, b);
  }
  WAM_DEV static uint4 gelu8(float4 lo, float4 hi, uint4 b) {
    return make_uint4(pack_bf2(gelu_f(lo.x + bf_lo(b.x)), gelu_f(lo.y + bf_hi(b.x))),
                      pack_bf2(gelu_f(lo.z + bf_lo(b.y)), gelu_f(lo.w + bf_hi(b.y))),
                      pack_bf2(gelu_f(hi.x + bf_lo(b.z)), gelu_f(hi.y + bf_hi(b.z))),
                      pack_bf2(gelu_f(hi.z + bf_lo(b.w)), gelu_f(hi.w + bf_hi(b.w))));
  }
};

// Epilogues with a bf16 output that can store eight consecutive columns of a
// row at once (pre8 / fin8: one 16-byte store where fin4 makes an 8-byte one).
template <class E>
struct Out8 {
  static constexpr bool value = false;
};
template <>
struct Out8<EpiGelu<bf16_t>> {
  static constexpr bool value = true;
};
template <>
struct Out8<EpiQKV<bf16_t>> {
  static constexpr bool value = true;
};

