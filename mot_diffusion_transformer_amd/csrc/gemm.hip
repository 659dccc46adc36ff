// GEMMs of the MoT world-action-model forward pass, all of the form
//   acc[m][n] = sum_k A[m][k] W[n][k]     (A activations, W = weight [out][in])
// followed by a per-element epilogue (bias, GELU, gated residual, q|k|v
// scatter).  Three kernels:
//   * gemm_bf16_mfma  -- bf16 on MFMA 32x32x16, LDS-staged double-buffered
//                        tiles; the video expert (M = B*T_v tokens) and large
//                        action batches;
//   * gemm_skinny_bf16 -- M <= 64 rows (the action expert's 32/64 tokens):
//                        weight streaming, MFMA 16x16x32, each weight byte
//                        read once, deterministic split-K;
//   * gemm_f32_valu   -- float32 models (VALU, LDS tiles).
#include "kernels.h"

// ============================================================================
// float32 VALU GEMM: 64x64 tile, BK 16, 256 threads, 4x4 outputs per thread.
// ============================================================================
template <class Epi>
__global__ void __launch_bounds__(256)
gemm_f32_valu(const float* __restrict__ A, int lda, const float* __restrict__ W, int ldw, int M, int N, int K,
              Epi epi) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sW[BK][BN + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int i = tid; i < BM * BK; i += 256) {
      int r = i / BK, c = i % BK;
      int gm = m0 + r, gk = k0 + c;
      sA[c][r] = (gm < M && gk < K) ? A[(size_t)gm * lda + gk] : 0.0f;
      int gn = n0 + r;
      sW[c][r] = (gn < N && gk < K) ? W[(size_t)gn * ldw + gk] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sW[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < M && n < N) epi(m, n, acc[i][j]);
    }
}

// ============================================================================
// bf16 MFMA GEMM.  Block tile BM x BN x 64, WM x WN wavefronts, each owning a
// (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles.  Global -> registers
// -> LDS, double-buffered: the next K tile is fetched while the current one
// feeds the MFMAs.  LDS rows are padded to 72 elements (144 B) so the
// 16-byte fragment reads of 32 consecutive rows hit distinct banks.
// Requires K % 64 == 0; M and N may be ragged.
// ============================================================================
template <int BM, int BN, int WM, int WN, class Epi>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_bf16_mfma(const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ W, int ldw, int M, int N, int K,
               int tiles_m, int tiles_n, Epi epi) {
  constexpr int BK = 64, LDK = BK + 8, NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int CPR = BK / 8;  // 16-byte chunks per tile row
  constexpr int A_LD = BM * CPR / NT, B_LD = BN * CPR / NT;
  static_assert(TM >= 1 && TN >= 1 && A_LD >= 1 && B_LD >= 1, "tile shape");
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Tile order: consecutive workgroups are dealt round-robin to the 8 XCDs;
  // remap so each XCD gets a contiguous band of tiles (shared A rows / W
  // columns stay in that XCD's L2), then walk the band column-major within
  // groups of 8 M-tiles.
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if (ntiles % 8 == 0) bid = (bid % 8) * (ntiles / 8) + bid / 8;
  const int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int gid = bid / group_size;
  const int first_m = gid * GROUP;
  const int gm_rows = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (bid % group_size) % gm_rows;
  const int tn = (bid % group_size) / gm_rows;
  const int m0 = tm * BM, n0 = tn * BN;

  uint4 ra[A_LD], rb[B_LD];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      int c = tid + i * NT, r = c / CPR, cc = c % CPR;
      int gm = m0 + r;
      ra[i] = gm < M ? *(const uint4*)(A + (size_t)gm * lda + k0 + cc * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      int c = tid + i * NT, r = c / CPR, cc = c % CPR;
      int gn = n0 + r;
      rb[i] = gn < N ? *(const uint4*)(W + (size_t)gn * ldw + k0 + cc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      int c = tid + i * NT, r = c / CPR, cc = c % CPR;
      *(uint4*)(&sA[buf][r * LDK + cc * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      int c = tid + i * NT, r = c / CPR, cc = c % CPR;
      *(uint4*)(&sB[buf][r * LDK + cc * 8]) = rb[i];
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int KT = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const bf16_t* a_s = sA[cur];
    const bf16_t* b_s = sB[cur];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        int row = wm * WTM + i * 32 + (lane & 31);
        af[i] = *(const bf16x8_t*)(a_s + row * LDK + kk * 16 + (lane >> 5) * 8);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int row = wn * WTN + j * 32 + (lane & 31);
        bfr[j] = *(const bf16x8_t*)(b_s + row * LDK + kk * 16 + (lane >> 5) * 8);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int m = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        int n = n0 + wn * WTN + j * 32 + (lane & 31);
        if (m < M && n < N) epi(m, n, acc[i][j][r]);
      }
}

// ============================================================================
// Weight-streaming GEMM for M <= 16*MT rows (MT <= 4).
// Workgroup = 4 wavefronts = 16 output columns (16 weight rows) x one K range.
// Wave w takes the 128-wide K chunks w, w+4, ... of that range; lane l
// (group g = l/16, r = l%16) streams 64 contiguous bytes of weight row
// n0 + r per chunk (k = chunk*128 + 32g .. +31) and the same k of the
// activation rows.  The MFMA k slots of lane group g are these 32 k values
// in four 8-wide steps; A and B use the same assignment, so the product is
// exact.  Partial sums of the 4 waves are added in LDS in wave order; with
// a K split across workgroups (gridDim.y > 1) each split writes its
// partial to `part` and gemm_splitk_reduce adds them in split order.
// ============================================================================
template <int MT, class Epi>
__global__ void __launch_bounds__(256)
gemm_skinny_bf16(const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ W, int ldw, int M, int N, int K,
                 int chunks_per_split, float* __restrict__ part, Epi epi) {
  __shared__ float red[4][MT][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int n0 = blockIdx.x * 16;
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int nchunks = K / 128;
  const int c_beg = split * chunks_per_split;
  const int c_end = min(nchunks, c_beg + chunks_per_split);
  const int wrow = n0 + r;
  const bool wok = wrow < N;
  const bf16_t* wp = W + (size_t)(wok ? wrow : 0) * ldw + g * 32;

  f32x4_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int c = c_beg + wave; c < c_end; c += 4) {
    const int k = c * 128;
    uint4 w4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w4[q] = wok ? *(const uint4*)(wp + k + q * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int arow = mt * 16 + r;
      uint4 a4[4];
      const bf16_t* ap = A + (size_t)arow * lda + k + g * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) a4[q] = arow < M ? *(const uint4*)(ap + q * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a4[q]),
                                                          __builtin_bit_cast(bf16x8_t, w4[q]), acc[mt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][mt][e][lane] = acc[mt][e];
  __syncthreads();
  if (wave != 0) return;
  // 16x16 accumulator layout: lane l, register e holds row 4*(l/16) + e, column l%16.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s = ((red[0][mt][e][lane] + red[1][mt][e][lane]) + red[2][mt][e][lane]) + red[3][mt][e][lane];
      const int m = mt * 16 + g * 4 + e, n = n0 + r;
      if (m < M && n < N) {
        if (nsplit == 1)
          epi(m, n, s);
        else
          part[((size_t)split * M + m) * N + n] = s;
      }
    }
}

template <class Epi>
__global__ void gemm_splitk_reduce(const float* __restrict__ part, int nsplit, int M, int N, Epi epi) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * N) return;
  float s = part[i];
  for (int sp = 1; sp < nsplit; ++sp) s += part[(size_t)sp * M * N + i];
  epi(i / N, i % N, s);
}

// Split plan of the skinny kernel: a function of (N, K) only, so a given
// shape always runs the same reduction order.
struct SkinnyPlan {
  int ntiles, nsplit, chunks_per_split;
};
static SkinnyPlan skinny_plan(int N, int K) {
  SkinnyPlan p;
  p.ntiles = (N + 15) / 16;
  const int nchunks = K / 128;
  int want = (512 + p.ntiles - 1) / p.ntiles;  // aim for >= 512 workgroups
  int cap = nchunks / 4 > 0 ? nchunks / 4 : 1;  // keep every wave of a split busy
  int ks = want < cap ? want : cap;
  if (ks < 1) ks = 1;
  p.chunks_per_split = (nchunks + ks - 1) / ks;
  p.nsplit = (nchunks + p.chunks_per_split - 1) / p.chunks_per_split;
  return p;
}

static bool use_skinny(int M, int K) { return M <= 64 && K % 128 == 0; }

size_t gemm_ws_floats(bool bf16, int M, int N, int K) {
  if (!bf16 || !use_skinny(M, K)) return 0;
  SkinnyPlan p = skinny_plan(N, K);
  return p.nsplit > 1 ? (size_t)p.nsplit * M * N : 0;
}

template <int BM, int BN, int WM, int WN, class Epi>
static hipError_t run_mfma(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K, const Epi& epi,
                           hipStream_t s) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  gemm_bf16_mfma<BM, BN, WM, WN, Epi><<<tm * tn, WM * WN * 64, 0, s>>>(A, lda, W, ldw, M, N, K, tm, tn, epi);
  return hipGetLastError();
}

template <class Epi>
static hipError_t gemm_bf16(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K, const Epi& epi,
                            float* ws, hipStream_t s) {
  if (use_skinny(M, K)) {
    SkinnyPlan p = skinny_plan(N, K);
    dim3 grid(p.ntiles, p.nsplit);
    float* part = p.nsplit > 1 ? ws : nullptr;
    if (M <= 16)
      gemm_skinny_bf16<1, Epi><<<grid, 256, 0, s>>>(A, lda, W, ldw, M, N, K, p.chunks_per_split, part, epi);
    else if (M <= 32)
      gemm_skinny_bf16<2, Epi><<<grid, 256, 0, s>>>(A, lda, W, ldw, M, N, K, p.chunks_per_split, part, epi);
    else
      gemm_skinny_bf16<4, Epi><<<grid, 256, 0, s>>>(A, lda, W, ldw, M, N, K, p.chunks_per_split, part, epi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    gemm_splitk_reduce<Epi><<<(M * N + 255) / 256, 256, 0, s>>>(ws, p.nsplit, M, N, epi);
    return hipGetLastError();
  }
  if (K % 64) return hipErrorInvalidValue;
  return run_mfma<128, 128, 2, 2>(A, lda, W, ldw, M, N, K, epi, s);
}

template <class T, class Epi>
hipError_t launch_gemm(const T* A, int lda, const T* W, int ldw, int M, int N, int K, const Epi& epi, float* ws,
                       hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    return gemm_bf16<Epi>(A, lda, W, ldw, M, N, K, epi, ws, s);
  } else {
    dim3 grid((N + 63) / 64, (M + 63) / 64);
    gemm_f32_valu<Epi><<<grid, 256, 0, s>>>(A, lda, W, ldw, M, N, K, epi);
    return hipGetLastError();
  }
}

#define WAM_INST_GEMM(T)                                                                                           \
  template hipError_t launch_gemm<T, EpiF32<T>>(const T*, int, const T*, int, int, int, int, const EpiF32<T>&,     \
                                                float*, hipStream_t);                                              \
  template hipError_t launch_gemm<T, EpiQKV<T>>(const T*, int, const T*, int, int, int, int, const EpiQKV<T>&,     \
                                                float*, hipStream_t);                                              \
  template hipError_t launch_gemm<T, EpiGateRes<T>>(const T*, int, const T*, int, int, int, int,                   \
                                                    const EpiGateRes<T>&, float*, hipStream_t);                    \
  template hipError_t launch_gemm<T, EpiGelu<T>>(const T*, int, const T*, int, int, int, int, const EpiGelu<T>&,   \
                                                 float*, hipStream_t);
WAM_INST_GEMM(float)
WAM_INST_GEMM(bf16_t)
