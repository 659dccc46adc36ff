// Softmax attention over two concatenated key segments, the operation at the
// centre of the Mixture-of-Transformers coupling: the video expert attends
// over its own tokens (segment 1 empty); the action expert's block i
// attends over [own keys ; video block i keys].  No mask, scale 1/sqrt(dh).
//
// bf16 path: LDS-tiled online softmax on MFMA 16x16x32.  Each wavefront owns
// 16 queries.  Scores are computed transposed, S^T = K Q^T, so each lane
// ends up holding 16 scores of ONE query (its column); those probabilities
// are exactly the B operand of O^T += V^T P^T, so P never leaves registers.
// V^T comes from LDS, where each key tile is stored transposed ([d][key]).
// Long key ranges with few query tiles (the action expert: 32-64 queries
// against ~2-4k keys) are split over workgroups; the partial (max, sum,
// unnormalised output) triples are merged in split order by a second kernel.
//
// float32 path: one wavefront per query, online softmax over 64-key chunks.
#include "kernels.h"

#include <math.h>

constexpr float kLog2e = 1.4426950408889634f;

template <class T>
WAM_DEV const T* key_row(const T* seg0, const T* seg1, int L0, int j, int dh) {
  return j < L0 ? seg0 + (size_t)j * dh : seg1 + (size_t)(j - L0) * dh;
}

// ============================================================================
// bf16 MFMA attention.  grid: (query tiles, B*H, splits); QW wavefronts.
// ============================================================================
template <int DH, int QW>
__global__ void __launch_bounds__(QW * 64)
attn_bf16_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k0, const bf16_t* __restrict__ v0, int L0,
               const bf16_t* __restrict__ k1, const bf16_t* __restrict__ v1, int L1, int H, int Tq,
               int tiles_per_split, float scale_log2, bf16_t* __restrict__ o, float* __restrict__ part) {
  constexpr int KT = 64;           // keys per tile
  constexpr int LDK = DH + 8;      // sK row stride (elements)
  constexpr int LDV = KT + 8;      // sV row stride (elements)
  constexpr int NTH = QW * 64;
  __shared__ __attribute__((aligned(16))) bf16_t sK[KT * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t sV[DH * LDV];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int L = L0 + L1;
  const int ntiles = (L + KT - 1) / KT;
  const int split = blockIdx.z, nsplit = gridDim.z;
  const int t_beg = split * tiles_per_split;
  const int t_end = min(ntiles, t_beg + tiles_per_split);

  const bf16_t* K0 = k0 + (size_t)bh * L0 * DH;
  const bf16_t* V0 = v0 + (size_t)bh * L0 * DH;
  const bf16_t* K1 = L1 > 0 ? k1 + (size_t)bh * L1 * DH : nullptr;
  const bf16_t* V1 = L1 > 0 ? v1 + (size_t)bh * L1 * DH : nullptr;

  // this lane's query (B operand column) and its fragments, kept in registers
  const int qi = blockIdx.x * (16 * QW) + wave * 16 + c16;
  const bool qok = qi < Tq;
  bf16x8_t qf[DH / 32];
  {
    const bf16_t* qp = q + ((size_t)bh * Tq + (qok ? qi : 0)) * DH + g * 8;
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) {
      uint4 u = qok ? *(const uint4*)(qp + ks * 32) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8_t, u);
    }
  }

  f32x4_t oacc[DH / 16];
#pragma unroll
  for (int i = 0; i < DH / 16; ++i) oacc[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  for (int tile = t_beg; tile < t_end; ++tile) {
    const int j0 = tile * KT;
    __syncthreads();  // the previous tile is fully consumed
    for (int c = threadIdx.x; c < KT * (DH / 8); c += NTH) {
      const int kr = c / (DH / 8), d8 = (c % (DH / 8)) * 8;
      const int j = j0 + kr;
      uint4 ku = make_uint4(0, 0, 0, 0), vu = make_uint4(0, 0, 0, 0);
      if (j < L) {
        ku = *(const uint4*)(key_row(K0, K1, L0, j, DH) + d8);
        vu = *(const uint4*)(key_row(V0, V1, L0, j, DH) + d8);
      }
      *(uint4*)(sK + kr * LDK + d8) = ku;
      const uint32_t w[4] = {vu.x, vu.y, vu.z, vu.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sV[(d8 + 2 * e) * LDV + kr] = (bf16_t)(w[e] & 0xFFFF);
        sV[(d8 + 2 * e + 1) * LDV + kr] = (bf16_t)(w[e] >> 16);
      }
    }
    __syncthreads();

    // S^T tile: 4 sub-tiles of 16 keys; lane holds keys jt*16 + 4g + e of query c16.
    f32x4_t s[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      s[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      const bf16_t* kp = sK + (jt * 16 + c16) * LDK + g * 8;
#pragma unroll
      for (int ks = 0; ks < DH / 32; ++ks)
        s[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8_t*)(kp + ks * 32), qf[ks], s[jt], 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + jt * 16 + 4 * g + e;
        float v = j < L ? s[jt][e] * scale_log2 : -INFINITY;
        s[jt][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);  // finite: every tile holds >= 1 real key
    const float alpha = exp2f(m_run - m_new);
    float ls = 0.0f;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = exp2f(s[jt][e] - m_new);
        s[jt][e] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * alpha + ls;
    m_run = m_new;

    // P^T fragments: k slot (g, e) of step ks <-> key (2ks + e/4)*16 + 4g + e%4.
    bf16x8_t pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 u;
      u.x = pack_bf2(s[2 * ks][0], s[2 * ks][1]);
      u.y = pack_bf2(s[2 * ks][2], s[2 * ks][3]);
      u.z = pack_bf2(s[2 * ks + 1][0], s[2 * ks + 1][1]);
      u.w = pack_bf2(s[2 * ks + 1][2], s[2 * ks + 1][3]);
      pf[ks] = __builtin_bit_cast(bf16x8_t, u);
    }
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      oacc[dt] *= alpha;
      const bf16_t* vp = sV + (dt * 16 + c16) * LDV + 4 * g;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint2 lo = *(const uint2*)(vp + ks * 32);
        uint2 hi = *(const uint2*)(vp + ks * 32 + 16);
        uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, u), pf[ks], oacc[dt], 0, 0, 0);
      }
    }
  }

  if (!qok) return;
  // O^T layout: lane holds d = dt*16 + 4g + e of query c16.
  if (nsplit == 1) {
    const float inv = 1.0f / l_run;
    bf16_t* op = o + ((size_t)b * Tq + qi) * (H * DH) + h * DH + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      uint2 u;
      u.x = pack_bf2(oacc[dt][0] * inv, oacc[dt][1] * inv);
      u.y = pack_bf2(oacc[dt][2] * inv, oacc[dt][3] * inv);
      *(uint2*)(op + dt * 16) = u;
    }
  } else {
    // partial record [bh][split][query][DH + 4]: unnormalised o, then (m, l, -, -)
    float* pp = part + (((size_t)bh * nsplit + split) * Tq + qi) * (DH + 4);
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
      *(float4*)(pp + dt * 16 + 4 * g) = make_float4(oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
    if (g == 0) {
      pp[DH] = m_run;
      pp[DH + 1] = l_run;
    }
  }
}

// Merge split partials in split order: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
template <class T>
__global__ void attn_merge(const float* __restrict__ part, int nsplit, int H, int Tq, int dh, T* __restrict__ o) {
  const int bh = blockIdx.y, qi = blockIdx.x;
  const int b = bh / H, h = bh - b * H;
  const size_t rec = (size_t)(dh + 4);
  const float* base = part + ((size_t)bh * nsplit * Tq + qi) * rec;
  const size_t sstride = (size_t)Tq * rec;
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, base[sp * sstride + dh]);
  float l = 0.0f;
  for (int sp = 0; sp < nsplit; ++sp) l += exp2f(base[sp * sstride + dh] - M) * base[sp * sstride + dh + 1];
  const float inv = 1.0f / l;
  for (int d = threadIdx.x; d < dh; d += blockDim.x) {
    float acc = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) acc += exp2f(base[sp * sstride + dh] - M) * base[sp * sstride + d];
    o[((size_t)b * Tq + qi) * (H * dh) + h * dh + d] = from_f32<T>(acc * inv);
  }
}

// ============================================================================
// float32 attention: one wavefront per query; 64-key chunks, lane j scores
// key j0 + j, then lanes own output features d = lane, lane + 64.
// ============================================================================
__global__ void __launch_bounds__(256)
attn_f32(const float* __restrict__ q, const float* __restrict__ k0, const float* __restrict__ v0, int L0,
         const float* __restrict__ k1, const float* __restrict__ v1, int L1, int H, int Tq, int dh, float scale,
         float* __restrict__ o) {
  const int lane = threadIdx.x & 63;
  const int qi = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int bh = blockIdx.y;
  if (qi >= Tq) return;
  const int b = bh / H, h = bh - b * H;
  const int L = L0 + L1;
  const float* K0 = k0 + (size_t)bh * L0 * dh;
  const float* V0 = v0 + (size_t)bh * L0 * dh;
  const float* K1 = L1 > 0 ? k1 + (size_t)bh * L1 * dh : nullptr;
  const float* V1 = L1 > 0 ? v1 + (size_t)bh * L1 * dh : nullptr;
  const float* qp = q + ((size_t)bh * Tq + qi) * dh;
  float m_run = -INFINITY, l_run = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
  for (int j0 = 0; j0 < L; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j < L) {
      const float* kp = key_row(K0, K1, L0, j, dh);
      float d = 0.0f;
      for (int e = 0; e < dh; ++e) d = fmaf(qp[e], kp[e], d);
      s = d * scale;
    }
    const float m_new = fmaxf(m_run, wave_max(s));
    const float alpha = expf(m_run - m_new);
    const float p = j < L ? expf(s - m_new) : 0.0f;
    l_run = l_run * alpha + wave_sum(p);
    acc0 *= alpha;
    acc1 *= alpha;
    const int n = min(64, L - j0);
    for (int jj = 0; jj < n; ++jj) {
      const float pj = __shfl(p, jj, 64);
      const float* vp = key_row(V0, V1, L0, j0 + jj, dh);
      if (lane < dh) acc0 = fmaf(pj, vp[lane], acc0);
      if (lane + 64 < dh) acc1 = fmaf(pj, vp[lane + 64], acc1);
    }
    m_run = m_new;
  }
  float* op = o + ((size_t)b * Tq + qi) * (H * dh) + h * dh;
  if (lane < dh) op[lane] = acc0 / l_run;
  if (lane + 64 < dh) op[lane + 64] = acc1 / l_run;
}

// ============================================================================
// launch plan: a function of the shape only (so results never depend on timing)
// ============================================================================
struct AttnPlan {
  int qw, qtiles, nsplit, tiles_per_split;
};
static AttnPlan attn_plan(int B, int H, int Tq, int L) {
  AttnPlan p;
  p.qw = Tq <= 32 ? 2 : 4;
  p.qtiles = (Tq + 16 * p.qw - 1) / (16 * p.qw);
  const int ntiles = (L + 63) / 64;
  const int base = B * H * p.qtiles;
  int want = base >= 256 ? 1 : (256 + base - 1) / base;
  if (want > ntiles) want = ntiles;
  if (want < 1) want = 1;
  p.tiles_per_split = (ntiles + want - 1) / want;
  p.nsplit = (ntiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

size_t attention_ws_floats(bool bf16, int B, int H, int dh, int Tq, int L0, int L1) {
  if (!bf16) return 0;
  AttnPlan p = attn_plan(B, H, Tq, L0 + L1);
  return p.nsplit > 1 ? (size_t)B * H * p.nsplit * Tq * (dh + 4) : 0;
}

template <int DH, int QW>
static void run_attn(const AttnPlan& p, const bf16_t* q, const bf16_t* k0, const bf16_t* v0, int L0, const bf16_t* k1,
                     const bf16_t* v1, int L1, int B, int H, int Tq, bf16_t* o, float* ws, hipStream_t s) {
  dim3 grid(p.qtiles, B * H, p.nsplit);
  const float scale_log2 = kLog2e / sqrtf((float)DH);
  attn_bf16_mfma<DH, QW><<<grid, QW * 64, 0, s>>>(q, k0, v0, L0, k1, v1, L1, H, Tq, p.tiles_per_split, scale_log2,
                                                   o, p.nsplit > 1 ? ws : nullptr);
}

template <class T>
hipError_t launch_attention(const T* q, const T* k0, const T* v0, int L0, const T* k1, const T* v1, int L1, int B,
                            int H, int dh, int Tq, T* o, float* ws, hipStream_t s) {
  if (Tq <= 0 || B <= 0) return hipSuccess;
  if (L0 + L1 <= 0) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2) {
    AttnPlan p = attn_plan(B, H, Tq, L0 + L1);
    if (dh == 128) {
      if (p.qw == 2) run_attn<128, 2>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s);
      else run_attn<128, 4>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s);
    } else if (dh == 64) {
      if (p.qw == 2) run_attn<64, 2>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s);
      else run_attn<64, 4>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s);
    } else {
      return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    attn_merge<bf16_t><<<dim3(Tq, B * H), 64, 0, s>>>(ws, p.nsplit, H, Tq, dh, o);
    return hipGetLastError();
  } else {
    if (dh > 128) return hipErrorInvalidValue;
    dim3 grid((Tq + 3) / 4, B * H);
    attn_f32<<<grid, 256, 0, s>>>(q, k0, v0, L0, k1, v1, L1, H, Tq, dh, 1.0f / sqrtf((float)dh), o);
    return hipGetLastError();
  }
}

template hipError_t launch_attention<float>(const float*, const float*, const float*, int, const float*, const float*,
                                            int, int, int, int, int, float*, float*, hipStream_t);
template hipError_t launch_attention<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*, int, const bf16_t*,
                                             const bf16_t*, int, int, int, int, int, bf16_t*, float*, hipStream_t);
