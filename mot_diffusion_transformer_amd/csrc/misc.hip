// Memory-bound kernels of the MoT world-action-model forward pass: the
// time embedding, the batched t-MLP / adaLN GEMV, fused LayerNorm +
// modulation, the input upcast, the action input projection and the fused
// final layer + Euler step + endpoint map.
#include "kernels.h"

#include <math.h>

#include <algorithm>

// ----------------------------------------------------------------------------
// time embedding: computed in double (cos/sin of arguments up to 1000), then
// stored as float; 256 values per t, so the cost is nil.
// ----------------------------------------------------------------------------
__global__ void temb_kernel(TList ts, int dim, float* __restrict__ E) {
  const int half = dim / 2;
  const int j = blockIdx.x;
  const double t = (double)ts.t[j];
  for (int k = threadIdx.x; k < half; k += blockDim.x) {
    double f = exp(-log(10000.0) * (double)k / (double)half);
    double arg = 1000.0 * t * f;
    E[(size_t)j * dim + k] = (float)cos(arg);
    E[(size_t)j * dim + half + k] = (float)sin(arg);
  }
}

hipError_t launch_temb(const TList& ts, int dim, float* E, hipStream_t s) {
  if (ts.n <= 0) return hipSuccess;
  temb_kernel<<<ts.n, 128, 0, s>>>(ts, dim, E);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// GEMV over J <= 16 right-hand vectors, weights streamed once.
// One wavefront per weight row; each lane reads 8 consecutive elements per
// step (16 B for bf16), the J activations sit in LDS (act_in applied once).
// ----------------------------------------------------------------------------
constexpr int GEMV_JMAX = 16;

template <class T> struct Vec8;
template <> struct Vec8<bf16_t> {
  uint4 u;
  WAM_DEV void load(const bf16_t* p) { u = *(const uint4*)p; }
  WAM_DEV float get(int e) const {
    uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
    return (e & 1) ? bf_hi(w) : bf_lo(w);
  }
};
template <> struct Vec8<float> {
  float4 a, b;
  WAM_DEV void load(const float* p) {
    a = *(const float4*)p;
    b = *(const float4*)(p + 4);
  }
  WAM_DEV float get(int e) const {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return v[e];
  }
};

template <class T>
__global__ void __launch_bounds__(256)
gemv_kernel(const T* __restrict__ W, int N, int K, const float* __restrict__ X, int J, int act_in,
            const T* __restrict__ bias, int act_out, float* __restrict__ Y, int ldy) {
  extern __shared__ float sx[];  // [J][K]
  for (int i = threadIdx.x; i < J * K; i += blockDim.x) {
    float v = X[i];
    sx[i] = act_in == 1 ? silu_f(v) : v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int n = blockIdx.x * 4 + wave; n < N; n += gridDim.x * 4) {
    float acc[GEMV_JMAX];
#pragma unroll
    for (int j = 0; j < GEMV_JMAX; ++j) acc[j] = 0.0f;
    const T* wr = W + (size_t)n * K;
    for (int k = lane * 8; k < K; k += 512) {
      Vec8<T> w;
      w.load(wr + k);
#pragma unroll
      for (int j = 0; j < GEMV_JMAX; ++j) {
        if (j < J) {
          const float* xr = sx + j * K + k;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j] = fmaf(w.get(e), xr[e], acc[j]);
        }
      }
    }
    const float b = bias ? to_f32<T>(bias[n]) : 0.0f;
#pragma unroll
    for (int j = 0; j < GEMV_JMAX; ++j) {
      if (j < J) {
        float v = wave_sum(acc[j]) + b;
        if (act_out == 1) v = silu_f(v);
        if (lane == 0) Y[(size_t)j * ldy + n] = v;
      }
    }
  }
}

// The same product for J <= 3 vectors and K <= 512 * KC: each wavefront
// takes 4 weight rows at a time and requests all of their values (KC 16-byte
// chunks per lane and row) before any arithmetic, so a group of rows costs
// one memory round trip.  Per lane the products are summed in the same order
// as gemv_kernel.
template <class T, int KC, int JN>
__global__ void __launch_bounds__(256)
gemv_rows_kernel(const T* __restrict__ W, int N, int K, const float* __restrict__ X, int act_in,
                 const T* __restrict__ bias, int act_out, float* __restrict__ Y, int ldy) {
  extern __shared__ float sx[];  // [JN][K]
  for (int i = threadIdx.x; i < JN * K; i += blockDim.x) {
    float v = X[i];
    sx[i] = act_in == 1 ? silu_f(v) : v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int n0 = (blockIdx.x * 4 + wave) * 4; n0 < N; n0 += gridDim.x * 16) {
    Vec8<T> w[4][KC];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const T* wr = W + (size_t)min(n0 + r, N - 1) * K;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int k = c * 512 + lane * 8;
        if (k < K) w[r][c].load(wr + k);
      }
    }
    float acc[4][JN];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < JN; ++j) acc[r][j] = 0.0f;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k = c * 512 + lane * 8;
      if (k < K) {
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          const float* xr = sx + j * K + k;
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][j] = fmaf(w[r][c].get(e), xr[e], acc[r][j]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + r;
      const float b = (bias && n < N) ? to_f32<T>(bias[n]) : 0.0f;
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        float v = wave_sum(acc[r][j]) + b;
        if (act_out == 1) v = silu_f(v);
        if (lane == 0 && n < N) Y[(size_t)j * ldy + n] = v;
      }
    }
  }
}

template <class T, int KC>
static hipError_t launch_gemv_rows(const T* W, int N, int K, const float* X, int J, int act_in, const T* bias,
                                   int act_out, float* Y, int ldy, hipStream_t s) {
  int grid = (N + 15) / 16;
  if (grid > 4096) grid = 4096;
  const size_t lds = (size_t)J * K * sizeof(float);
  if (J == 1)
    gemv_rows_kernel<T, KC, 1><<<grid, 256, lds, s>>>(W, N, K, X, act_in, bias, act_out, Y, ldy);
  else if (J == 2)
    gemv_rows_kernel<T, KC, 2><<<grid, 256, lds, s>>>(W, N, K, X, act_in, bias, act_out, Y, ldy);
  else
    gemv_rows_kernel<T, KC, 3><<<grid, 256, lds, s>>>(W, N, K, X, act_in, bias, act_out, Y, ldy);
  return hipGetLastError();
}

// The same product for 4 <= J <= 16 vectors and bf16 weights on float32
// MFMA (16x16x4: float32 products and sums).  A wavefront owns 16 weight
// rows (16 output columns) at a time: operand A holds the J vectors (rows
// J..15 are zero), operand B the 16 weight rows.  Lane l (g = l / 16,
// r = l % 16) streams 32 contiguous bytes of weight row n0 + r per
// 64-wide k chunk, k = kb + 16 g .. kb + 16 g + 15; MFMA q of the chunk
// puts k = kb + 16 g + q in k-slot g of both operands, so every k is
// counted once.  Four chunks are in flight per wavefront.  The vectors'
// LDS rows are padded by 4 floats: the 16 lanes of one 16-byte read then
// touch all 64 banks once.
__global__ void __launch_bounds__(256)
gemv_mfma_bf16(const bf16_t* __restrict__ W, int N, int K, const float* __restrict__ X, int J, int act_in,
               const bf16_t* __restrict__ bias, int act_out, float* __restrict__ Y, int ldy) {
  extern __shared__ float sx[];  // [J][K + 4]
  const int KP = K + 4;
  for (int i = threadIdx.x; i < J * K; i += blockDim.x) {
    const float v = X[i];
    sx[(i / K) * KP + i % K] = act_in == 1 ? silu_f(v) : v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int nch = K / 64;
  const bool live = r < J;
  const float* xr = sx + (size_t)(live ? r : 0) * KP + 16 * g;
  const int ntiles = (N + 15) / 16;
  for (int t = blockIdx.x * 4 + wave; t < ntiles; t += gridDim.x * 4) {
    const int n0 = t * 16;
    const bf16_t* wp = W + (size_t)min(n0 + r, N - 1) * K + 16 * g;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    uint4 wb[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < nch) {
        wb[u][0] = *(const uint4*)(wp + u * 64);
        wb[u][1] = *(const uint4*)(wp + u * 64 + 8);
      }
    for (int c0 = 0; c0 < nch; c0 += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u;
        if (c < nch) {
          const uint4 w0 = wb[u][0], w1 = wb[u][1];
          if (c + 4 < nch) {
            wb[u][0] = *(const uint4*)(wp + (c + 4) * 64);
            wb[u][1] = *(const uint4*)(wp + (c + 4) * 64 + 8);
          }
          const float4* xp = (const float4*)(xr + c * 64);
          const float4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
          const float xa[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
          const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const float b = (q & 1) ? bf_hi(ww[q >> 1]) : bf_lo(ww[q >> 1]);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(live ? xa[q] : 0.0f, b, acc, 0, 0, 0);
          }
        }
      }
    }
    // 16x16 accumulator layout: lane l, register e holds vector j = 4 (l / 16) + e, column n0 + l % 16
    const int n = n0 + r;
    if (n < N) {
      const float bn = bias ? to_f32<bf16_t>(bias[n]) : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * g + e;
        if (j < J) {
          float v = acc[e] + bn;
          if (act_out == 1) v = silu_f(v);
          Y[(size_t)j * ldy + n] = v;
        }
      }
    }
  }
}

template <class T>
hipError_t launch_gemv(const T* W, int N, int K, const float* X, int J, int act_in, const T* bias,
                       int act_out, float* Y, int ldy, hipStream_t s) {
  if (N <= 0 || J <= 0) return hipSuccess;
  if (J > GEMV_JMAX || K % 8 || J * K > 16384) return hipErrorInvalidValue;  // LDS <= 64 KB
  if constexpr (sizeof(T) == 2) {
    if (J >= 4 && K % 64 == 0 && (size_t)J * (K + 4) * sizeof(float) <= 65536) {
      const int ntiles = (N + 15) / 16;
      const int grid = std::min((ntiles + 3) / 4, 512);
      gemv_mfma_bf16<<<grid, 256, (size_t)J * (K + 4) * sizeof(float), s>>>(W, N, K, X, J, act_in, bias, act_out,
                                                                             Y, ldy);
      return hipGetLastError();
    }
  }
  if (J <= 3 && K <= 2048) {
    if (K <= 512) return launch_gemv_rows<T, 1>(W, N, K, X, J, act_in, bias, act_out, Y, ldy, s);
    if (K <= 1024) return launch_gemv_rows<T, 2>(W, N, K, X, J, act_in, bias, act_out, Y, ldy, s);
    if (K <= 1536) return launch_gemv_rows<T, 3>(W, N, K, X, J, act_in, bias, act_out, Y, ldy, s);
    return launch_gemv_rows<T, 4>(W, N, K, X, J, act_in, bias, act_out, Y, ldy, s);
  }
  int grid = (N + 3) / 4;
  if (grid > 4096) grid = 4096;
  gemv_kernel<T><<<grid, 256, (size_t)J * K * sizeof(float), s>>>(W, N, K, X, J, act_in, bias, act_out, Y, ldy);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// LayerNorm (population variance, no affine) + adaLN modulation.
// One wavefront per row, float4 chunks, two-pass statistics from registers.
// MAXC (float4 chunks per lane) is the smallest of 2/4/8/32 that holds the
// row, so narrow rows keep few registers and many waves per SIMD.
// ----------------------------------------------------------------------------
template <class T, int MAXC>
__global__ void __launch_bounds__(256)
ln_mod_kernel(const float* __restrict__ x, int rows, int d, const float* __restrict__ shift,
              const float* __restrict__ scale, float eps, T* __restrict__ h, int rows_per_group, size_t mod_stride) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  if (mod_stride) {  // per-sample modulation: row group g uses the g-th vectors
    shift += (size_t)(row / rows_per_group) * mod_stride;
    scale += (size_t)(row / rows_per_group) * mod_stride;
  }
  const float4* xr = (const float4*)(x + (size_t)row * d);
  const int nc = d / 4;
  // the row and its modulation vectors are requested together: one memory
  // round trip before the reductions instead of two (rows of up to 2048:
  // wider ones hold only the row, 128 registers, and read the modulation
  // where it is used)
  constexpr bool HOLD = MAXC <= 8;
  float4 v[MAXC], sh[HOLD ? MAXC : 1], sc[HOLD ? MAXC : 1];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    int c = lane + i * 64;
    if (c < nc) {
      v[i] = xr[c];
      if constexpr (HOLD) {
        sh[i] = ((const float4*)shift)[c];
        sc[i] = ((const float4*)scale)[c];
      }
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    int c = lane + i * 64;
    if (c < nc) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float mean = wave_sum(sum) / (float)d;
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    int c = lane + i * 64;
    if (c < nc) {
      float a = v[i].x - mean, b = v[i].y - mean, e = v[i].z - mean, f = v[i].w - mean;
      sq += (a * a + b * b) + (e * e + f * f);
    }
  }
  const float rstd = rsqrtf(wave_sum(sq) / (float)d + eps);
  T* hr = h + (size_t)row * d;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    int c = lane + i * 64;
    if (c < nc) {
      const float4 shc = HOLD ? sh[HOLD ? i : 0] : ((const float4*)shift)[c];
      const float4 scc = HOLD ? sc[HOLD ? i : 0] : ((const float4*)scale)[c];
      float o0 = (v[i].x - mean) * rstd * (1.0f + scc.x) + shc.x;
      float o1 = (v[i].y - mean) * rstd * (1.0f + scc.y) + shc.y;
      float o2 = (v[i].z - mean) * rstd * (1.0f + scc.z) + shc.z;
      float o3 = (v[i].w - mean) * rstd * (1.0f + scc.w) + shc.w;
      if constexpr (sizeof(T) == 2) {
        uint2 p;
        p.x = pack_bf2(o0, o1);
        p.y = pack_bf2(o2, o3);
        *(uint2*)(hr + 4 * c) = p;
      } else {
        *(float4*)(hr + 4 * c) = make_float4(o0, o1, o2, o3);
      }
    }
  }
}

// The same LayerNorm + modulation for rows of exactly NCH * 256 features
// (768 and 1536 in the workloads): lane l owns float4 chunks l + 64 i, every
// chunk exists, so the row and both modulation vectors are requested at once
// with no per-lane condition (with one, the compiler waited for each chunk's
// loads before the next: one memory round trip per chunk), and the two
// reductions run on DPP.
template <class T, int NCH>
__global__ void __launch_bounds__(256)
ln_mod_exact_kernel(const float* __restrict__ x, int rows, int d, const float* __restrict__ shift,
                    const float* __restrict__ scale, float eps, T* __restrict__ h, int rows_per_group,
                    size_t mod_stride) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wavefront
  if (mod_stride) {
    shift += (size_t)(row / rows_per_group) * mod_stride;
    scale += (size_t)(row / rows_per_group) * mod_stride;
  }
  const float4* xr = (const float4*)(x + (size_t)row * d) + lane;
  const float4* shr = (const float4*)shift + lane;
  const float4* scr = (const float4*)scale + lane;
  float4 v[NCH], sh[NCH], sc[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    v[i] = xr[64 * i];
    sh[i] = shr[64 * i];
    sc[i] = scr[64 * i];
  }
  // every load above is issued here, before the reductions (left alone, the
  // scheduler sinks the modulation loads past them: a second round trip)
  __builtin_amdgcn_sched_barrier(0);
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = wave_sum_dpp(sum) / (float)d;
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const float a = v[i].x - mean, b = v[i].y - mean, e = v[i].z - mean, f = v[i].w - mean;
    sq += (a * a + b * b) + (e * e + f * f);
  }
  const float rstd = rsqrtf(wave_sum_dpp(sq) / (float)d + eps);
  T* hr = h + (size_t)row * d + 4 * lane;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const float o0 = (v[i].x - mean) * rstd * (1.0f + sc[i].x) + sh[i].x;
    const float o1 = (v[i].y - mean) * rstd * (1.0f + sc[i].y) + sh[i].y;
    const float o2 = (v[i].z - mean) * rstd * (1.0f + sc[i].z) + sh[i].z;
    const float o3 = (v[i].w - mean) * rstd * (1.0f + sc[i].w) + sh[i].w;
    if constexpr (sizeof(T) == 2) {
      uint2 p;
      p.x = pack_bf2(o0, o1);
      p.y = pack_bf2(o2, o3);
      *(uint2*)(hr + 256 * i) = p;
    } else {
      *(float4*)(hr + 256 * i) = make_float4(o0, o1, o2, o3);
    }
  }
}

template <class T>
hipError_t launch_ln_mod(const float* x, int rows, int d, const float* shift, const float* scale, float eps,
                         T* h, hipStream_t s, int rows_per_group, size_t mod_stride) {
  if (rows <= 0) return hipSuccess;
  if (d % 4 || d > 4 * 64 * 32 || rows_per_group < 1) return hipErrorInvalidValue;
  const int grid = (rows + 3) / 4;
  if (d == 768) {
    ln_mod_exact_kernel<T, 3><<<grid, 256, 0, s>>>(x, rows, d, shift, scale, eps, h, rows_per_group, mod_stride);
    return hipGetLastError();
  }
  if (d == 1536) {
    ln_mod_exact_kernel<T, 6><<<grid, 256, 0, s>>>(x, rows, d, shift, scale, eps, h, rows_per_group, mod_stride);
    return hipGetLastError();
  }
  if (d <= 512)
    ln_mod_kernel<T, 2><<<grid, 256, 0, s>>>(x, rows, d, shift, scale, eps, h, rows_per_group, mod_stride);
  else if (d <= 1024)
    ln_mod_kernel<T, 4><<<grid, 256, 0, s>>>(x, rows, d, shift, scale, eps, h, rows_per_group, mod_stride);
  else if (d <= 2048)
    ln_mod_kernel<T, 8><<<grid, 256, 0, s>>>(x, rows, d, shift, scale, eps, h, rows_per_group, mod_stride);
  else
    ln_mod_kernel<T, 32><<<grid, 256, 0, s>>>(x, rows, d, shift, scale, eps, h, rows_per_group, mod_stride);
  return hipGetLastError();
}

// A feature pair (e, e+1) as one access of its raw bits.
template <class T> struct PairBits;
template <> struct PairBits<bf16_t> {
  using U = uint32_t;
  WAM_DEV static U ld(const bf16_t* p) { return *(const uint32_t*)p; }
  WAM_DEV static float lo(U u) { return bf_lo(u); }
  WAM_DEV static float hi(U u) { return bf_hi(u); }
  WAM_DEV static void st(bf16_t* p, float a, float b) { *(uint32_t*)p = pack_bf2(a, b); }
};
template <> struct PairBits<float> {
  using U = uint2;
  WAM_DEV static U ld(const float* p) { return *(const uint2*)p; }
  WAM_DEV static float lo(U u) { return __uint_as_float(u.x); }
  WAM_DEV static float hi(U u) { return __uint_as_float(u.y); }
  WAM_DEV static void st(float* p, float a, float b) { *(float2*)p = make_float2(a, b); }
};

// ----------------------------------------------------------------------------
// Block variant: QK-RMSNorm over all heads of a token, then (rope_w > 0) the
// 3-D rotary embedding, on q and k [B][H][T][dh] in place.  One wavefront per
// (tensor, sample, token); lane l owns the feature pairs l, l+64, ... of the
// token's H*dh/2 pairs (head = pair / (dh/2)), so every access is a 4-byte
// pair and a wave instruction covers 256 contiguous bytes of a head.  Since
// dh/2 divides 64, a lane holds the same pair index in every head, so its
// rotation angle is computed once per token.  The token's values stay in
// registers between the sum of squares and the output (PPL pairs per lane).
// The sum of squares, the gains and the rotation are float32.
// ----------------------------------------------------------------------------
template <class T, int PPL>
__global__ void __launch_bounds__(256)
qk_norm_rope_kernel(T* __restrict__ x0, const T* __restrict__ g0, T* __restrict__ x1, const T* __restrict__ g1,
                    int ntensors, int B, int H, int Tn, int dh, float eps, int rope_h, int rope_w) {
  const int lane = threadIdx.x & 63;
  // wavefront-uniform, and said so: otherwise the tensor (and whether it has
  // gains) counts as per-lane, the gain loads sit in an exec-masked branch,
  // and each one is waited for before the next (one memory round trip each)
  const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (item >= ntensors * B * Tn) return;
  const int which = item / (B * Tn), bt = item - which * (B * Tn);
  const int b = bt / Tn, t = bt - b * Tn;
  T* x = which == 0 ? x0 : x1;
  const T* g = which == 0 ? g0 : g1;
  const int np = dh / 2, npairs = H * np;
  const int e = 2 * (lane % np);          // this lane's feature pair within every head
  const int h0 = lane / np, hstep = 64 / np;  // its first head, and the head step between its pairs
  T* base = x + ((size_t)b * H * Tn + t) * dh + e;
  const size_t hstride = (size_t)Tn * dh;
  // Pair j of this lane is head h0 + hstep j (valid while below H).  Up to
  // 32 pairs per lane, its values and gains are requested at once,
  // unconditionally, from a head clamped to H - 1, and masked afterwards: a
  // load under a per-lane condition whose other lanes get a constant makes
  // the compiler wait for it before the next one.  More pairs would not fit
  // in registers that way; they are read under the condition.
  // Each pair is one access of its raw bits (a bf16 pair is one 32-bit
  // word), converted after the loads: loading the two halves as 16-bit
  // values made the compiler wait for each load to pack it into a register.
  constexpr bool PRE = PPL <= 32;
  typename PairBits<T>::U rx[PRE ? PPL : 1], rg[PRE ? PPL : 1];
  float va[PPL], vc[PPL];
  float gla[PRE ? PPL : 1], glc[PRE ? PPL : 1];
  if constexpr (PRE) {
#pragma unroll
    for (int j = 0; j < PPL; ++j) rx[j] = PairBits<T>::ld(base + (size_t)min(h0 + hstep * j, H - 1) * hstride);
    if (g) {  // uniform
#pragma unroll
      for (int j = 0; j < PPL; ++j) rg[j] = PairBits<T>::ld(g + min(h0 + hstep * j, H - 1) * dh + e);
    }
#pragma unroll
    for (int j = 0; j < PPL; ++j) {
      const bool ok = lane + 64 * j < npairs;
      va[j] = ok ? PairBits<T>::lo(rx[j]) : 0.0f;
      vc[j] = ok ? PairBits<T>::hi(rx[j]) : 0.0f;
      gla[j] = g ? PairBits<T>::lo(rg[j]) : 1.0f;
      glc[j] = g ? PairBits<T>::hi(rg[j]) : 1.0f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < PPL; ++j) {
      va[j] = vc[j] = 0.0f;
      if (lane + 64 * j < npairs) {
        const T* p = base + (size_t)(h0 + hstep * j) * hstride;
        va[j] = to_f32<T>(p[0]);
        vc[j] = to_f32<T>(p[1]);
      }
    }
  }
  float rstd = 1.0f;
  if (g) {
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < PPL; ++j) ss = fmaf(va[j], va[j], fmaf(vc[j], vc[j], ss));
    rstd = rsqrtf(wave_sum(ss) / (float)(2 * npairs) + eps);
  }
  float cs = 1.0f, sn = 0.0f;
  if (rope_w > 0) {
    // band (frame, row, column) of this pair, its index i in the band and the band size
    const int s0 = dh - 4 * (dh / 6), s1 = 2 * (dh / 6);
    int pos, i, size;
    if (e < s0) {
      pos = t / (rope_h * rope_w); i = e / 2; size = s0;
    } else if (e < s0 + s1) {
      pos = (t / rope_w) % rope_h; i = (e - s0) / 2; size = s1;
    } else {
      pos = t % rope_w; i = (e - s0 - s1) / 2; size = s1;
    }
    // angle = pos * 10000^(-2i/size) = pos * 2^(-log2(10000) 2i/size)
    sincosf((float)pos * exp2f(-13.287712379549449f * (float)(2 * i) / (float)size), &sn, &cs);
  }
#pragma unroll
  for (int j = 0; j < PPL; ++j) {
    if (lane + 64 * j < npairs) {
      const int hd = h0 + hstep * j;
      float a = va[j] * rstd, c = vc[j] * rstd;
      if (g) {
        a *= PRE ? gla[PRE ? j : 0] : to_f32<T>(g[hd * dh + e]);
        c *= PRE ? glc[PRE ? j : 0] : to_f32<T>(g[hd * dh + e + 1]);
      }
      PairBits<T>::st(base + (size_t)hd * hstride, a * cs - c * sn, a * sn + c * cs);
    }
  }
}

template <class T>
hipError_t launch_qk_norm_rope(T* q, const T* gq, T* k, const T* gk, int B, int H, int Tn, int dh, float eps,
                               int rope_h, int rope_w, hipStream_t s) {
  const int nt = k ? 2 : 1;
  if (B <= 0 || Tn <= 0) return hipSuccess;
  if (dh % 2 || 64 % (dh / 2) || (rope_w > 0 && (rope_h <= 0 || Tn % (rope_h * rope_w)))) return hipErrorInvalidValue;
  const int ppl = (H * dh / 2 + 63) / 64;  // pairs per lane
  const long long items = (long long)nt * B * Tn;
  const unsigned grid = (unsigned)((items + 3) / 4);
  if (ppl <= 8)
    qk_norm_rope_kernel<T, 8><<<grid, 256, 0, s>>>(q, gq, k, gk, nt, B, H, Tn, dh, eps, rope_h, rope_w);
  else if (ppl <= 16)
    qk_norm_rope_kernel<T, 16><<<grid, 256, 0, s>>>(q, gq, k, gk, nt, B, H, Tn, dh, eps, rope_h, rope_w);
  else if (ppl <= 32)
    qk_norm_rope_kernel<T, 32><<<grid, 256, 0, s>>>(q, gq, k, gk, nt, B, H, Tn, dh, eps, rope_h, rope_w);
  else if (ppl <= 128)
    qk_norm_rope_kernel<T, 128><<<grid, 256, 0, s>>>(q, gq, k, gk, nt, B, H, Tn, dh, eps, rope_h, rope_w);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
template hipError_t launch_qk_norm_rope<float>(float*, const float*, float*, const float*, int, int, int, int, float,
                                               int, int, hipStream_t);
template hipError_t launch_qk_norm_rope<bf16_t>(bf16_t*, const bf16_t*, bf16_t*, const bf16_t*, int, int, int, int,
                                                float, int, int, hipStream_t);

// ----------------------------------------------------------------------------
// upcast of the video tokens into the float32 residual stream
// ----------------------------------------------------------------------------
template <class T>
__global__ void to_f32_kernel(const T* __restrict__ src, size_t n, float* __restrict__ x) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) x[i] = to_f32<T>(src[i]);
}

template <class T>
hipError_t launch_to_f32(const T* src, size_t n, float* x, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  to_f32_kernel<T><<<(unsigned)blocks, 256, 0, s>>>(src, n, x);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// selective reuse across observations: which tokens moved, and the row
// gather / scatter of the active tokens
// ----------------------------------------------------------------------------
// One wavefront per token: float32 sums of (xn - xp)^2 and xp^2, then the flag.
template <class T>
__global__ void __launch_bounds__(256)
select_flags_kernel(const T* __restrict__ xn, const T* __restrict__ xp, int n_tok, int d, float tau2,
                    int* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= n_tok) return;
  const T* a = xn + (size_t)j * d;
  const T* b = xp + (size_t)j * d;
  float dd = 0.0f, pp = 0.0f;
  for (int k = lane; k < d; k += 64) {
    const float u = to_f32<T>(a[k]), w = to_f32<T>(b[k]);
    const float df = u - w;
    dd = fmaf(df, df, dd);
    pp = fmaf(w, w, pp);
  }
  dd = wave_sum(dd);
  pp = wave_sum(pp);
  if (lane == 0) flags[j] = dd > tau2 * pp ? 1 : 0;
}

// One workgroup: the flags in idx[0..n_tok) become, in place, the ascending
// indices of the flagged tokens.  Per 1024-token chunk every thread reads
// its flag before any write (an index lands at or before its own token, so
// no unread flag is overwritten); ballots give the ranks.
__global__ void __launch_bounds__(1024) compact_flags_kernel(int* __restrict__ idx, int n_tok, int* __restrict__ count) {
  __shared__ int wtot[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int base = 0;
  for (int c0 = 0; c0 < n_tok; c0 += 1024) {
    const int j = c0 + tid;
    const int f = j < n_tok ? idx[j] : 0;
    const unsigned long long mask = __ballot(f != 0);
    const int pre = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[w] = __popcll(mask);
    __syncthreads();
    int off = base, tot = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < w) off += wtot[i];
      tot += wtot[i];
    }
    if (f) idx[off + pre] = j;
    base += tot;
    __syncthreads();
  }
  if (tid == 0) count[0] = base;
}

template <class T>
hipError_t launch_select_tokens(const T* xn, const T* xp, int n_tok, int d, float tau2, int* idx, int* count,
                                hipStream_t s) {
  if (n_tok <= 0) return hipErrorInvalidValue;
  select_flags_kernel<T><<<(n_tok + 3) / 4, 256, 0, s>>>(xn, xp, n_tok, d, tau2, idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  compact_flags_kernel<<<1, 1024, 0, s>>>(idx, n_tok, count);
  return hipGetLastError();
}

template <class T>
__global__ void __launch_bounds__(256)
gather_rows_kernel(const T* __restrict__ src, const int* __restrict__ idx, int d, float* __restrict__ x) {
  const int r = blockIdx.x;
  const T* sp = src + (size_t)idx[r] * d;
  float* xp = x + (size_t)r * d;
  for (int k = threadIdx.x; k < d; k += 256) xp[k] = to_f32<T>(sp[k]);
}

template <class T>
hipError_t launch_gather_rows(const T* src, const int* idx, int n, int d, float* x, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  gather_rows_kernel<T><<<n, 256, 0, s>>>(src, idx, d, x);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256)
scatter_rows_kernel(const float* __restrict__ x, const int* __restrict__ idx, int d, float* __restrict__ dst) {
  const int r = blockIdx.x;
  const float* xp = x + (size_t)r * d;
  float* dp = dst + (size_t)idx[r] * d;
  for (int k = threadIdx.x; k < d; k += 256) dp[k] = xp[k];
}

hipError_t launch_scatter_rows(const float* x, const int* idx, int n, int d, float* dst, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  scatter_rows_kernel<<<n, 256, 0, s>>>(x, idx, d, dst);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// action input projection y0 = a W_in^T + b_in (K = action_dim <= 64)
// ----------------------------------------------------------------------------
template <class T>
__global__ void action_in_kernel(const float* __restrict__ a, int M, int A, const T* __restrict__ W,
                                 const T* __restrict__ b, int d, float* __restrict__ y) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * d) return;
  int m = i / d, n = i - m * d;
  float acc = 0.0f;
  for (int k = 0; k < A; ++k) acc = fmaf(a[m * A + k], to_f32<T>(W[(size_t)n * A + k]), acc);
  y[i] = acc + to_f32<T>(b[n]);
}

template <class T>
hipError_t launch_action_in(const float* a, int M, int A, const T* W, const T* b, int d, float* y, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  action_in_kernel<T><<<(M * d + 255) / 256, 256, 0, s>>>(a, M, A, W, b, d, y);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// final layer + Euler step + endpoint map, one action token per workgroup
// ----------------------------------------------------------------------------
// NY, KPL > 0 (d <= 256 NY, d <= 64 KPL): this thread's row elements c =
// threadIdx.x + 256 i and, for the wavefront's first OB outputs (o = wave +
// 4 j), lane `lane`'s weights c = lane + 64 i are held in registers.  The
// kernel is a chain of dependent steps over 32-row inputs, so all of them,
// with the modulation, biases and previous actions, are requested at its
// start: the loads are unconditional, from clamped addresses, and the
// values out of range are masked where they are used (a load under a
// per-lane condition whose other lanes get a constant makes the compiler
// wait for it before the next one).  NY = KPL = 0: read from memory where
// used (any d).  The sums run in the same order either way.
template <class T, int NY, int KPL>
__global__ void __launch_bounds__(256)
final_euler_kernel(const float* __restrict__ y, int d, const float* __restrict__ modf,
                   const T* __restrict__ W_out, const T* __restrict__ b_out, int A, float eps,
                   const float* a, float dt, float t, float* a_next, float* __restrict__ v_out,
                   float* __restrict__ f_out, int rows_per_group, size_t mod_stride, TList t_g, TList dt_g) {
  extern __shared__ float sh[];  // [d] normalised row, then 8 reduction slots
  float* red = sh + d;
  const int m = blockIdx.x;
  if (mod_stride) {  // per-sample times and final modulation: row group g uses the g-th
    const int gi = m / rows_per_group;
    modf += (size_t)gi * mod_stride;
    t = t_g.t[gi];
    dt = dt_g.t[gi];
  }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float* yr = y + (size_t)m * d;
  constexpr bool REG = NY > 0;
  constexpr int OB = REG ? 4 : 1;
  float yv[REG ? NY : 1], shv[REG ? NY : 1], scv[REG ? NY : 1];
  T wv[OB][REG ? KPL : 1], bv[OB];
  float av[OB];
  auto load_outputs = [&](int o0) {
#pragma unroll
    for (int j = 0; j < OB; ++j) {
      const int o = min(o0 + 4 * j, A - 1);
      const T* wr = W_out + (size_t)o * d;
#pragma unroll
      for (int i = 0; i < KPL; ++i) wv[j][i] = wr[min(lane + 64 * i, d - 1)];
      bv[j] = b_out[o];
      av[j] = a[(size_t)m * A + o];
    }
  };
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < NY; ++i) {
      const int c = min((int)threadIdx.x + 256 * i, d - 1);
      yv[i] = yr[c];
      shv[i] = modf[c];
      scv[i] = modf[d + c];
    }
    load_outputs(wave);
  }
  auto yat = [&](int i) { return REG ? yv[i] : yr[threadIdx.x + 256 * i]; };
  const int ny = REG ? NY : (d + 255) / 256;
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < ny; ++i)
    if (threadIdx.x + 256 * i < d) s += yat(i);
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  const float mean = ((red[0] + red[1]) + (red[2] + red[3])) / (float)d;
  float q = 0.0f;
#pragma unroll
  for (int i = 0; i < ny; ++i)
    if (threadIdx.x + 256 * i < d) {
      const float e = yat(i) - mean;
      q += e * e;
    }
  q = wave_sum(q);
  if (lane == 0) red[4 + wave] = q;
  __syncthreads();
  const float rstd = rsqrtf(((red[4] + red[5]) + (red[6] + red[7])) / (float)d + eps);
#pragma unroll
  for (int i = 0; i < ny; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < d) {
      const float shift = REG ? shv[i] : modf[c], scale = REG ? scv[i] : modf[d + c];
      sh[c] = (yat(i) - mean) * rstd * (1.0f + scale) + shift;
    }
  }
  __syncthreads();
  auto finish = [&](int o, float acc, float bias, float aprev) {
    const float v = acc + bias;
    const size_t idx = (size_t)m * A + o;
    if (v_out) v_out[idx] = v;
    if (f_out) f_out[idx] = fmaf(-t, v, aprev);
    a_next[idx] = fmaf(-dt, v, aprev);
  };
  if constexpr (REG) {
    for (int o0 = wave; o0 < A; o0 += 4 * OB) {
      if (o0 != wave) load_outputs(o0);
      float acc[OB];
#pragma unroll
      for (int j = 0; j < OB; ++j) {
        acc[j] = 0.0f;
#pragma unroll
        for (int i = 0; i < KPL; ++i)
          if (lane + 64 * i < d) acc[j] = fmaf(sh[lane + 64 * i], to_f32<T>(wv[j][i]), acc[j]);
      }
#pragma unroll
      for (int j = 0; j < OB; ++j) acc[j] = wave_sum(acc[j]);
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < OB; ++j)
          if (o0 + 4 * j < A) finish(o0 + 4 * j, acc[j], to_f32<T>(bv[j]), av[j]);
      }
    }
  } else {
    for (int o = wave; o < A; o += 4) {
      const T* wr = W_out + (size_t)o * d;
      float acc = 0.0f;
      for (int c = lane; c < d; c += 64) acc = fmaf(sh[c], to_f32<T>(wr[c]), acc);
      acc = wave_sum(acc);
      if (lane == 0) finish(o, acc, to_f32<T>(b_out[o]), a[(size_t)m * A + o]);
    }
  }
}

template <class T>
hipError_t launch_final_euler(const float* y, int M, int d, const float* modf, const T* W_out, const T* b_out,
                              int A, float eps, const float* a, float dt, float t, float* a_next, float* v_out,
                              float* f_out, hipStream_t s, int rows_per_group, size_t mod_stride, const TList* t_g,
                              const TList* dt_g) {
  if (M <= 0) return hipSuccess;
  if (rows_per_group < 1 || (mod_stride && (!t_g || !dt_g || (M + rows_per_group - 1) / rows_per_group > t_g->n)))
    return hipErrorInvalidValue;
  TList none{};
  // row elements per thread and weights per lane held in registers, by width
  auto kern = d <= 768    ? final_euler_kernel<T, 3, 12>
              : d <= 2048 ? final_euler_kernel<T, 8, 32>
                          : final_euler_kernel<T, 0, 0>;
  kern<<<M, 256, (size_t)(d + 8) * sizeof(float), s>>>(y, d, modf, W_out, b_out, A, eps, a, dt, t, a_next, v_out,
                                                       f_out, rows_per_group, mod_stride, t_g ? *t_g : none,
                                                       dt_g ? *dt_g : none);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// teacher-anchored targets: a_t = (1 - t_g) a0 + t_g eps, and after the
// teacher's rollout u = (a_t - a) / t_g, with the time t_g of row group g
// (one group = one rollout's T_a x A values)
// ----------------------------------------------------------------------------
__global__ void targets_init_kernel(const float* __restrict__ a0, const float* __restrict__ eps, int n, int per_group,
                                    TList tg, float* __restrict__ a_t, float* __restrict__ a_t_copy) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float t = tg.t[i / per_group];
  const float v = fmaf(t, eps[i], (1.0f - t) * a0[i]);
  a_t[i] = v;
  if (a_t_copy) a_t_copy[i] = v;
}

__global__ void targets_u_kernel(const float* __restrict__ a_t, const float* __restrict__ a, int n, int per_group,
                                 TList tg, float* __restrict__ u) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  u[i] = (a_t[i] - a[i]) / tg.t[i / per_group];
}

hipError_t launch_targets_init(const float* a0, const float* eps, int n, int per_group, const TList& tg, float* a_t,
                               float* a_t_copy, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (per_group < 1 || (n + per_group - 1) / per_group > tg.n) return hipErrorInvalidValue;
  targets_init_kernel<<<(n + 255) / 256, 256, 0, s>>>(a0, eps, n, per_group, tg, a_t, a_t_copy);
  return hipGetLastError();
}

hipError_t launch_targets_u(const float* a_t, const float* a, int n, int per_group, const TList& tg, float* u,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (per_group < 1 || (n + per_group - 1) / per_group > tg.n) return hipErrorInvalidValue;
  targets_u_kernel<<<(n + 255) / 256, 256, 0, s>>>(a_t, a, n, per_group, tg, u);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Debug delay: one wavefront waits `ticks` of the 100 MHz real-time counter,
// sleeping between reads; the loop is also capped at 2^20 rounds (each
// s_sleep 8 is >= 512 clocks), so the kernel always ends.
__global__ void __launch_bounds__(64) delay_kernel(uint32_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t i = 0; i < (1u << 20); ++i) {
    if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(8);
  }
}

hipError_t launch_delay(uint32_t us, hipStream_t s) {
  if (us == 0) return hipSuccess;
  delay_kernel<<<1, 64, 0, s>>>(std::min<uint32_t>(us, kMaxDebugDelayUs) * 100u);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
#define WAM_INST_MISC(T)                                                                                   \
  template hipError_t launch_gemv<T>(const T*, int, int, const float*, int, int, const T*, int, float*, int, \
                                     hipStream_t);                                                          \
  template hipError_t launch_ln_mod<T>(const float*, int, int, const float*, const float*, float, T*,       \
                                       hipStream_t, int, size_t);                                           \
  template hipError_t launch_to_f32<T>(const T*, size_t, float*, hipStream_t);                              \
  template hipError_t launch_select_tokens<T>(const T*, const T*, int, int, float, int*, int*, hipStream_t); \
  template hipError_t launch_gather_rows<T>(const T*, const int*, int, int, float*, hipStream_t);           \
  template hipError_t launch_action_in<T>(const float*, int, int, const T*, const T*, int, float*,         \
                                          hipStream_t);                                                     \
  template hipError_t launch_final_euler<T>(const float*, int, int, const float*, const T*, const T*, int,  \
                                            float, const float*, float, float, float*, float*, float*,      \
                                            hipStream_t, int, size_t, const TList*, const TList*);
WAM_INST_MISC(float)
WAM_INST_MISC(bf16_t)
