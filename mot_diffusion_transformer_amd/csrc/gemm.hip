// GEMMs of the MoT world-action-model forward pass, all of the form
//   acc[m][n] = sum_k A[m][k] W[n][k]     (A activations, W = weight [out][in])
// followed by an epilogue (bias, GELU, gated residual, q|k|v scatter).
// Three kernels:
//   * gemm_bf16_lds   -- bf16 on MFMA 32x32x16, tiles streamed into LDS by
//                        direct global->LDS loads; the video expert
//                        (M = B*T_v tokens) and large action batches;
//   * gemm_skinny_bf16 -- M <= 64 rows (the action expert's 32/64 tokens):
//                        weight streaming, MFMA 16x16x32, each weight byte
//                        read once, deterministic split-K;
//   * gemm_f32_valu   -- float32 models (VALU, LDS tiles).
#include "kernels.h"

#include <type_traits>

#include <algorithm>

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
// bf16 MFMA GEMM, multi-stage LDS pipeline fed by direct global->LDS loads.
//
// Block tile BM x BN x 64, WM x WN wavefronts, each owning a (BM/WM) x (BN/WN)
// sub-tile of 32x32 MFMA tiles.  Each K tile is brought into LDS by
// buffer_load_dwordx4 ... lds (no VGPR staging): a wavefront instruction writes
// 64 x 16 B contiguous LDS bytes, so the bank-conflict-avoiding layout is
// produced on the global side: LDS slot s of tile row r holds the 16-byte
// k-chunk c = s ^ ((r >> 1) & 7) (an XOR swizzle), and fragment reads undo
// it.  gfx950 serves a 16-byte-per-lane LDS read 16 lanes (256 B) at a time;
// the 16 rows those lanes read then cover all 64 banks once.
// STAGES tiles are in flight; the wait for tile k+1 (vmcnt) leaves the
// STAGES-2 tiles issued after it loading under the MFMAs.  The barrier
// between tiles is a plain s_barrier behind explicit waits: a
// __syncthreads() fence would wait for every load in flight.
// Rows past M (columns past N) read row M-1 (N-1) instead: they only feed
// outputs that are never stored.  Requires K % 64 == 0.
// K split across workgroups: blockIdx.y = s takes K range [s klen, (s+1) klen)
// (gridDim.y splits); with more than one split the epilogue is EpiPart and
// gemm_splitk_reduce4 adds the partial tiles in split order.
// ============================================================================

template <int N>
WAM_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  // gfx9 s_waitcnt: vmcnt[3:0] and [15:14], expcnt[6:4] = 7, lgkmcnt[11:8] = 15
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Wait until at most `ahead` tiles (LOADS wave instructions each) are still
// loading: s_waitcnt takes an immediate, so the depth is unrolled.
template <int LOADS, int MAXA>
WAM_DEV void wait_tiles_ahead(int ahead) {
  if constexpr (MAXA == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= MAXA) wait_vmcnt<MAXA * LOADS>();
    else wait_tiles_ahead<LOADS, MAXA - 1>(ahead);
  }
}
WAM_DEV void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt 0, vmcnt/expcnt untouched
WAM_DEV void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM, int BN, int WM, int WN, int STAGES, class Epi>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_bf16_lds(const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ W, int ldw, int M, int N, int K,
              int klen, int tiles_m, int tiles_n, Epi epi) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int ROWS = BM + BN;               // tile rows of A then W, 128 B each
  constexpr int STAGE_BYTES = ROWS * 128;
  constexpr int GT = ROWS * 8 / 64;           // wave instructions (1 KB, 8 rows each) per stage
  constexpr int LOADS = (GT + NW - 1) / NW;   // per wave; when NW does not divide GT, the last
                                              // LOADS * NW - GT of them repeat the first ones
                                              // (same source, same LDS bytes: a harmless rewrite)
  static_assert(TM >= 1 && TN >= 1, "tile shape");
  static_assert(ROWS % 8 == 0 && LOADS * NW - GT <= GT, "stage rows");
  static_assert(LOADS * (STAGES - 1) < 64, "vmcnt range");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

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

  // Tiles are fetched with buffer_load ... lds through buffer descriptors
  // (MUBUF, not FLAT: with a FLAT load writing LDS in flight the compiler
  // can only wait for all LDS reads at once, which would serialise the
  // fragment pipeline below).  Per lane a fixed byte offset of its row and
  // 16-byte chunk; the K position goes in the scalar offset.  Each wave
  // instruction covers 8 whole tile rows, so it reads A or W uniformly.
  const BufRsrc rs_a = buf_rsrc(A, (uint32_t)(((size_t)(M - 1) * lda + K) * 2));
  const BufRsrc rs_w = buf_rsrc(W, (uint32_t)(((size_t)(N - 1) * ldw + K) * 2));
  uint32_t voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int g0 = wave * LOADS + i, g = g0 < GT ? g0 : g0 - GT;  // wave instruction of the stage
    const int P = g * 64 + lane;  // 16-byte slot within the stage
    const int r = P >> 3, c = (P & 7) ^ ((r >> 1) & 7);
    if (r < BM) voff[i] = (uint32_t)(((size_t)min(m0 + r, M - 1) * lda + c * 8) * 2);
    else voff[i] = (uint32_t)(((size_t)min(n0 + (r - BM), N - 1) * ldw + c * 8) * 2);
  }
  auto issue = [&](int stage, int k0) {
    unsigned char* base = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int g0 = wave * LOADS + i, g = g0 < GT ? g0 : g0 - GT;
      const bool is_a = g * 8 < BM;
      buf_load_lds16(is_a ? rs_a : rs_w, base + g * 1024, voff[i], (uint32_t)k0 * 2);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // this workgroup's K tiles: [kbase, kbase + KT)
  const int KT = klen / 64;
  const int kbase = blockIdx.y * klen;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s, kbase + s * 64);

  // fragment row offsets (bytes) and swizzle keys
  int a_off[TM], b_off[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_off[i] = (wm * WTM + i * 32 + (lane & 31)) * 128;
#pragma unroll
  for (int j = 0; j < TN; ++j) b_off[j] = (BM + wn * WTN + j * 32 + (lane & 31)) * 128;
  const int key = (lane >> 1) & 7;  // (row >> 1) & 7 for every fragment row (rows are 32-aligned + lane % 32)
  const int hi = lane >> 5;

  // Software pipeline, fragments double-buffered in registers: the reads of
  // k-step kk+1 are issued before the MFMAs of step kk.  Each tile ends by
  // issuing its last MFMAs ahead of the wait for the next tile and the
  // barrier, so they run while the wavefront waits and while the next
  // tile's first fragments are read.  The scheduling groups and the
  // scheduling barrier pin that order; left alone the compiler sinks each
  // read next to its MFMA and serialises the two.
  bf16x8_t af[2][TM], bfr[2][TN];
  auto frag = [&](int buf, const unsigned char* st, int kk) {
    const int slot = ((2 * kk + hi) ^ key) * 16;
#pragma unroll
    for (int i = 0; i < TM; ++i) af[buf][i] = *(const bf16x8_t*)(st + a_off[i] + slot);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[buf][j] = *(const bf16x8_t*)(st + b_off[j] + slot);
  };
  auto mfma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][j], acc[i][j], 0, 0, 0);
  };

  wait_tiles_ahead<LOADS, STAGES - 2>(min(STAGES - 2, KT - 1));
  // no scalar load may be pending in the loop: those return out of order,
  // and the compiler would then wait for every LDS read, not just the oldest
  wait_lgkmcnt0();
  block_barrier();
  // The loads of tile kt+STAGES-1 are issued during tile kt, a few between
  // the MFMAs of each of its first SPREAD k-steps: all of them at once right
  // after the barrier would queue every wavefront's requests at the address
  // unit together and hold the wavefronts at the issue.  With two stages the
  // next tile is waited for at the end of this one, so they all go first.
  constexpr int SPREAD = STAGES > 2 ? 4 : 1;
  constexpr int LPS = (LOADS + SPREAD - 1) / SPREAD;  // loads per k-step
  auto issue_part = [&](int stage, int k0, auto partc) {
    constexpr int lo = decltype(partc)::value * LPS, hi = lo + LPS < LOADS ? lo + LPS : LOADS;
    unsigned char* base = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int i = lo; i < hi; ++i) {
      const int g0 = wave * LOADS + i, g = g0 < GT ? g0 : g0 - GT;
      const bool is_a = g * 8 < BM;
      buf_load_lds16(is_a ? rs_a : rs_w, base + g * 1024, voff[i], (uint32_t)k0 * 2);
    }
  };
  // one K tile; LOAD: also issue tile kt+STAGES-1 (which exists)
  auto tile = [&](int kt, auto loadc) {
    constexpr bool LOAD = decltype(loadc)::value;
    const unsigned char* st = smem + (kt % STAGES) * STAGE_BYTES;
    // stage (kt-1) % STAGES: every read of it finished before the last barrier
    const int ls = (kt + STAGES - 1) % STAGES, lk = kbase + (kt + STAGES - 1) * 64;
    frag(0, st, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);  // the reads of step 0 first
    auto step = [&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      constexpr int nl = LOAD && kk < SPREAD ? (kk * LPS + LPS < LOADS ? LPS : (LOADS > kk * LPS ? LOADS - kk * LPS : 0)) : 0;
      if constexpr (kk < 3) frag((kk + 1) & 1, st, kk + 1);
      if constexpr (nl > 0) issue_part(ls, lk, kkc);
      mfma(kk & 1);
      if constexpr (SPREAD == 1 && nl > 0) __builtin_amdgcn_sched_group_barrier(0x020, nl, 0);  // all loads first
      if constexpr (kk < 3) __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);  // DS reads of step kk+1
      if constexpr (SPREAD == 1) {
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
      } else {
        // the MFMAs of step kk, one load after each of the first nl
        static_for<TM * TN>([&](auto jc) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if constexpr (decltype(jc)::value < nl) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        });
        if constexpr (nl > TM * TN) __builtin_amdgcn_sched_group_barrier(0x020, nl - TM * TN, 0);
      }
    };
    static_for<4>(step);
    __builtin_amdgcn_sched_barrier(0);
  };
  int kt = 0;
  for (; kt + STAGES - 1 < KT; ++kt) {
    tile(kt, std::true_type{});
    // tile kt+1 has landed once the STAGES-2 tiles issued after it are the
    // only ones loading; this wavefront's reads of stage kt are complete
    // (lgkmcnt 0) before the barrier lets another wavefront refill it
    wait_vmcnt<(STAGES - 2) * LOADS>();
    wait_lgkmcnt0();
    block_barrier();
  }
  for (; kt < KT; ++kt) {
    tile(kt, std::false_type{});
    if (kt + 1 < KT) {
      wait_tiles_ahead<LOADS, STAGES - 2>(min(STAGES - 2, KT - 2 - kt));
      wait_lgkmcnt0();
      block_barrier();
    }
  }

  // Epilogue through LDS: each wavefront stages one 32-row slab of its
  // accumulators at a time (row stride WTN + 8 floats: the two half-waves
  // land on disjoint banks), then reads it back row-wise so every lane owns
  // four consecutive columns: vector loads of bias/gate/residual and 8- or
  // 16-byte stores instead of one scalar access per element.
  constexpr int ES = WTN + 8;
  static_assert(NW * 32 * ES * 4 <= STAGES * STAGE_BYTES, "epilogue staging must fit in the pipeline LDS");
  wait_vmcnt<0>();
  block_barrier();  // every wavefront is done with the pipeline buffers
  Epi ep = epi;
  epi_split(ep, blockIdx.y);
  float* eb = (float*)smem + wave * 32 * ES;
  constexpr int LPR = WTN / 4;         // float4 chunks per staged row
  constexpr int CHUNKS = 32 * LPR;     // per slab
  static_assert(CHUNKS % 64 == 0 && (8 * WTN) % 64 == 0, "epilogue lane mapping");
  const int nw_lo = n0 + wn * WTN, nw_hi = min(nw_lo + WTN, N);
  // 4 consecutive columns per lane; epilogues whose 4 columns are not
  // contiguous in memory (value columns of a q|k|v projection) go per element
  const bool row_path = (N % 4) == 0 && epi_rows_ok(ep, nw_lo, nw_hi);
  // value columns of a q|k|v projection (stored transposed, tokens
  // contiguous) read the slab by columns instead: four consecutive rows of
  // one column per lane, one 8-byte store along the transposed row
  const bool col_path = epi_cols_ok(ep, nw_lo);
  // one slab per accumulator row block; unrolled at compile time (a loop
  // the compiler could not unroll would index the accumulators at run time,
  // out of scratch memory)
  auto slab = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) eb[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * ES + j * 32 + (lane & 31)] = acc[i][j][r];
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    const int mb = m0 + wm * WTM + i * 32;
    // Each path below first issues the loads of every group it will store
    // (pre4: bias, gate, residual), then does the arithmetic and the stores
    // (fin4), so the slab's loads take one memory round trip, not one each.
    if (col_path) {
      constexpr int NPC = 8 * WTN / 64;
      Pre4 pc[NPC];
#pragma unroll
      for (int p = 0; p < NPC; ++p) {
        const int c = p * 64 + lane;
        const int col = c >> 3, r4 = (c & 7) * 4;  // 8 lanes cover one column's 32 rows
        // unconditional, from a clamped column: a load under a per-lane
        // condition would again wait before the next one
        pc[p] = epi_preT4(ep, min(mb + r4, M - 1), min(nw_lo + col, N - 1));
      }
#pragma unroll
      for (int p = 0; p < NPC; ++p) {
        const int c = p * 64 + lane;
        const int col = c >> 3, r4 = (c & 7) * 4;
        const float4 v = make_float4(eb[r4 * ES + col], eb[(r4 + 1) * ES + col], eb[(r4 + 2) * ES + col],
                                     eb[(r4 + 3) * ES + col]);
        const int m = mb + r4, n = nw_lo + col;
        if (n < N) {
          if (m + 3 < M) {
            epi_finT4(ep, m, n, v, pc[p]);
          } else {
            if (m < M) ep(m, n, v.x);
            if (m + 1 < M) ep(m + 1, n, v.y);
            if (m + 2 < M) ep(m + 2, n, v.z);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
      return;
    }
    // (a flag, not a `continue`: with one the slab loop is not unrolled and
    // the accumulators go to scratch)
    const bool row8 = Out8<Epi>::value && row_path && (N % 8) == 0;
    if constexpr (Out8<Epi>::value) {
      // bf16 outputs: eight consecutive columns per lane, one 16-byte store
      // (half the store instructions of the four-column path)
      if (row8) {  // uniform; every clamped group of eight lies inside the row
        constexpr int LPR8 = WTN / 8, CH8 = 32 * LPR8;
        static_assert(CH8 % 64 == 0, "epilogue lane mapping");
        uint4 pb[CH8 / 64];
#pragma unroll
        for (int p = 0; p < CH8 / 64; ++p) {
          const int c = p * 64 + lane;
          const int row = c / LPR8, c8 = (c % LPR8) * 8;
          pb[p] = ep.pre8(min(mb + row, M - 1), min(nw_lo + c8, N - 8));
        }
#pragma unroll
        for (int p = 0; p < CH8 / 64; ++p) {
          const int c = p * 64 + lane;
          const int row = c / LPR8, c8 = (c % LPR8) * 8;
          const float4 lo = *(const float4*)(eb + row * ES + c8), hi = *(const float4*)(eb + row * ES + c8 + 4);
          const int m = mb + row, n = nw_lo + c8;
          if (m < M) {
            if (n + 7 < N) {
              ep.fin8(m, n, lo, hi, pb[p]);
            } else {
              const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (n + e < N) ep(m, n + e, v[e]);
            }
          }
        }
      }
    }
    Pre4 pr[CHUNKS / 64];
    if (row_path && !row8) {  // uniform; then N % 4 == 0, so every clamped group of four lies inside the row
#pragma unroll
      for (int p = 0; p < CHUNKS / 64; ++p) {
        const int c = p * 64 + lane;
        const int row = c / LPR, c4 = (c % LPR) * 4;
        // unconditional, from a clamped position (only used where it is the
        // real one): a load under a per-lane condition would again wait
        pr[p] = ep.pre4(min(mb + row, M - 1), min(nw_lo + c4, N - 4));
      }
    }
    if (!row8) {
#pragma unroll
      for (int p = 0; p < CHUNKS / 64; ++p) {
        const int c = p * 64 + lane;
        const int row = c / LPR, c4 = (c % LPR) * 4;
        const float4 v = *(const float4*)(eb + row * ES + c4);
        const int m = mb + row, n = nw_lo + c4;
        if (m < M) {
          if (row_path && n + 3 < N) {
            ep.fin4(m, n, v, pr[p]);
          } else {
            if (n < N) ep(m, n, v.x);
            if (n + 1 < N) ep(m, n + 1, v.y);
            if (n + 2 < N) ep(m, n + 2, v.z);
            if (n + 3 < N) ep(m, n + 3, v.w);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  };
  static_for<TM>(slab);
}

template <int BM, int BN, int WM, int WN, int STAGES, class Epi>
static hipError_t run_lds(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K, const Epi& epi,
                          hipStream_t s, int nsplit = 1) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  // buffer offsets and record counts are 32-bit
  if (((size_t)(M - 1) * lda + K) * 2 >= (1ull << 31) || ((size_t)(N - 1) * ldw + K) * 2 >= (1ull << 31))
    return hipErrorInvalidValue;
  if (nsplit < 1 || (K / 64) % nsplit) return hipErrorInvalidValue;
  const int klen = K / nsplit;
  const size_t lds = (size_t)STAGES * (BM + BN) * 128;
  auto kern = gemm_bf16_lds<BM, BN, WM, WN, STAGES, Epi>;
  static bool attr_set = false;  // per instantiation; the attribute is process-wide
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  kern<<<dim3(tm * tn, nsplit), WM * WN * 64, lds, s>>>(A, lda, W, ldw, M, N, K, klen, tm, tn, epi);
  return hipGetLastError();
}

// Sum of the nsplit partial [M][N] tiles in split order, then the epilogue;
// four consecutive columns per thread (N % 4 == 0).
template <class Epi>
__global__ void __launch_bounds__(256)
gemm_splitk_reduce4(const float* __restrict__ part, int nsplit, int M, int N, Epi epi) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const size_t mn = (size_t)M * N;
  if ((size_t)i * 4 >= mn) return;
  float4 v = ((const float4*)part)[i];
  for (int sp = 1; sp < nsplit; ++sp) v = add4(v, ((const float4*)(part + sp * mn))[i]);
  const int m = (int)(((size_t)i * 4) / N), n = (int)(((size_t)i * 4) % N);
  if (epi_rows_ok(epi, n, n + 4)) {
    epi.store4(m, n, v);
  } else {
    epi(m, n, v.x);
    epi(m, n + 1, v.y);
    epi(m, n + 2, v.z);
    epi(m, n + 3, v.w);
  }
}

// One tile configuration, K unsplit or split over nsplit workgroups with the
// partial tiles in ws (nsplit * M * N floats).
template <int BM, int BN, int WM, int WN, int STAGES, class Epi>
static hipError_t run_tiled(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K, const Epi& epi,
                            int nsplit, float* ws, hipStream_t s) {
  if (nsplit == 1) return run_lds<BM, BN, WM, WN, STAGES, Epi>(A, lda, W, ldw, M, N, K, epi, s);
  if (!ws || N % 4) return hipErrorInvalidValue;
  hipError_t e = run_lds<BM, BN, WM, WN, STAGES, EpiPart>(A, lda, W, ldw, M, N, K, EpiPart{ws, N, (size_t)M * N},
                                                          s, nsplit);
  if (e != hipSuccess || std::is_same<Epi, EpiPart>::value) return e;  // EpiPart: the partials are the result
  const size_t n4 = (size_t)M * N / 4;
  gemm_splitk_reduce4<Epi><<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(ws, nsplit, M, N, epi);
  return hipGetLastError();
}

// ============================================================================
// Weight-streaming GEMM for M <= 16*MT rows (MT <= 4).
// Workgroup = WAVES (4 or 8) wavefronts = 16 output columns (16 weight rows)
// x one K range; 8 when a range has more than 4 chunks, so that every chunk
// is requested at once.  Wave w takes the 128-wide K chunks w, w+WAVES, ...
// of that range; lane l
// (group g = l/16, r = l%16) streams 64 contiguous bytes of weight row
// n0 + r per chunk (k = chunk*128 + 32g .. +31) and the same k of the
// activation rows.  The MFMA k slots of lane group g are these 32 k values
// in four 8-wide steps; A and B use the same assignment, so the product is
// exact.  Partial sums of the waves are added in LDS in wave order; with
// a K split across workgroups (gridDim.y > 1) each split writes its
// partial to `part` and gemm_splitk_reduce adds them in split order.
// ============================================================================
template <int MT, class Epi, int WAVES = 4>
__global__ void __launch_bounds__(WAVES * 64)
gemm_skinny_bf16(const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ W, int ldw, int M, int N, int K,
                 int chunks_per_split, float* __restrict__ part, Epi epi) {
  __shared__ float red[WAVES][MT][4][64];
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

  for (int c = c_beg + wave; c < c_end; c += WAVES) {
    const int k = c * 128;
    // the chunk's weight and activation fragments are all requested before
    // any is used, from clamped rows (zeros put in afterwards): one memory
    // round trip per chunk
    uint4 w4[4], a4[MT][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w4[q] = *(const uint4*)(wp + k + q * 8);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16_t* ap = A + (size_t)min(mt * 16 + r, M - 1) * lda + k + g * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) a4[mt][q] = *(const uint4*)(ap + q * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (!wok) w4[q] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (mt * 16 + r >= M) a4[mt][q] = make_uint4(0, 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a4[mt][q]),
                                                          __builtin_bit_cast(bf16x8_t, w4[q]), acc[mt], 0, 0, 0);
      }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][mt][e][lane] = acc[mt][e];
  // 16x16 accumulator layout: lane l, register e holds row 4*(l/16) + e,
  // column l%16.  The tile's outputs go out in groups of four, one group per
  // thread over all the wavefronts (one wavefront doing every element would
  // run MT x 4 chains of dependent accesses in a row): four consecutive rows
  // of one column for the transposed value columns of a q|k|v projection,
  // else four consecutive columns of one row.  Each sum adds the
  // wavefronts' partials in wave order.  The epilogue's own loads (bias,
  // gate, residual) are issued before the barrier, from clamped positions,
  // so they arrive while the partials are exchanged.
  constexpr int NG = MT * 64;
  const int gi = threadIdx.x, mt = gi >> 6, l = gi & 63;
  const bool one = nsplit == 1;
  const bool col_path = one && epi_cols_ok(epi, n0);
  const bool row_path = !col_path && (N % 4) == 0 && epi_rows_ok(epi, n0, min(n0 + 16, N));
  Pre4 pre{};
  if (gi < NG && one) {  // uniform per wavefront (NG is a multiple of 64)
    if (col_path) pre = epi_preT4(epi, min(mt * 16 + 4 * (l >> 4), M - 1), min(n0 + (l & 15), N - 1));
    else if (row_path) pre = epi.pre4(min(mt * 16 + (l >> 2), M - 1), min(n0 + 4 * (l & 3), N - 4));
  }
  __syncthreads();
  if (gi >= NG) return;
  if (col_path) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s = red[0][mt][e][l];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) s += red[w][mt][e][l];
      v[e] = s;
    }
    const int m = mt * 16 + 4 * (l >> 4), n = n0 + (l & 15);
    if (n < N) {
      if (m + 3 < M) {
        epi_finT4(epi, m, n, make_float4(v[0], v[1], v[2], v[3]), pre);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (m + e < M) epi(m + e, n, v[e]);
      }
    }
    return;
  }
  const int rr = l >> 2, c4 = 4 * (l & 3);
  float4 v = *(const float4*)&red[0][mt][rr & 3][(rr >> 2) * 16 + c4];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) v = add4(v, *(const float4*)&red[w][mt][rr & 3][(rr >> 2) * 16 + c4]);
  const int m = mt * 16 + rr, n = n0 + c4;
  if (m >= M) return;
  if (!one) {
    float* pp = part + ((size_t)split * M + m) * N + n;
    if ((N % 4) == 0 && n + 3 < N) {
      *(float4*)pp = v;
    } else {
      if (n < N) pp[0] = v.x;
      if (n + 1 < N) pp[1] = v.y;
      if (n + 2 < N) pp[2] = v.z;
      if (n + 3 < N) pp[3] = v.w;
    }
  } else if (row_path && n + 3 < N) {
    epi.fin4(m, n, v, pre);
  } else {
    if (n < N) epi(m, n, v.x);
    if (n + 1 < N) epi(m, n + 1, v.y);
    if (n + 2 < N) epi(m, n + 2, v.z);
    if (n + 3 < N) epi(m, n + 3, v.w);
  }
}

// Sum of the nsplit partial [M][N] tiles in split order, then the epilogue.
// The weight-streaming GEMMs' tiles are small (M <= 64), so few threads run
// and each one's latency counts: up to SB partials are requested at once
// (guards uniform across the workgroup, so no load waits for another).
template <class Epi>
__global__ void gemm_splitk_reduce(const float* __restrict__ part, int nsplit, int M, int N, Epi epi) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * N) return;
  constexpr int SB = 8;
  float s = 0.0f;
  for (int b = 0; b < nsplit; b += SB) {
    float p[SB];
#pragma unroll
    for (int k = 0; k < SB; ++k)
      if (b + k < nsplit) p[k] = part[(size_t)(b + k) * M * N + i];  // uniform
#pragma unroll
    for (int k = 0; k < SB; ++k)
      if (b + k < nsplit) s = b + k == 0 ? p[k] : s + p[k];
  }
  epi(i / N, i % N, s);
}

// Split reduction of the weight-streaming GEMM with the gated residual,
// followed in the same kernel by the LayerNorm + modulation the next GEMM
// needs (rows of d = NCH * 256 features, one wavefront per row):
//   x[m] += gate (sum_s part_s[m] + bias)   -- the sum in split order, as
//                                              gemm_splitk_reduce + EpiGateRes
//   h[m] = LN(x[m]) (1 + scale) + shift      -- as ln_mod_exact_kernel
// Every input of the row (partials, residual, gate, bias, modulation) is
// requested at once: one memory round trip, where the two kernels it
// replaces take a launch and two; the statistics reduce on DPP.
template <class T, int NCH, int MAXS>
__global__ void __launch_bounds__(256)
splitk_gateres_ln_kernel(const float* __restrict__ part, int nsplit, int M, int d, EpiGateRes<T> epi,
                         const float* __restrict__ shift, const float* __restrict__ scale, float eps,
                         T* __restrict__ h, int rows_per_group, size_t mod_stride) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // uniform per wavefront
  const size_t mn = (size_t)M * d;
  const float* pr = part + (size_t)row * d + 4 * lane;
  float* xr = epi.x + (size_t)row * epi.ldx + 4 * lane;
  const float* gr = epi.g_row(row) + 4 * lane;
  const T* br = epi.bias + 4 * lane;
  const size_t moff = mod_stride ? (size_t)(row / rows_per_group) * mod_stride : 0;
  const float* shr = shift + moff + 4 * lane;
  const float* scr = scale + moff + 4 * lane;
  float4 ps[MAXS][NCH];
  uint4 xv[NCH], gv[NCH], bv[NCH], shv[NCH], scv[NCH];
#pragma unroll
  for (int sp = 0; sp < MAXS; ++sp)
    if (sp < nsplit)  // uniform
#pragma unroll
      for (int i = 0; i < NCH; ++i) ps[sp][i] = *(const float4*)(pr + sp * mn + 256 * i);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    xv[i] = Raw4<float>::ld(xr + 256 * i);
    gv[i] = Raw4<float>::ld(gr + 256 * i);
    bv[i] = Raw4<T>::ld(br + 256 * i);
    shv[i] = Raw4<float>::ld(shr + 256 * i);
    scv[i] = Raw4<float>::ld(scr + 256 * i);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is in flight before the first use
  float4 y[NCH];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    float4 acc = ps[0][i];
#pragma unroll
    for (int sp = 1; sp < MAXS; ++sp)
      if (sp < nsplit) acc = add4(acc, ps[sp][i]);
    const float4 x = Raw4<float>::f(xv[i]), g = Raw4<float>::f(gv[i]), b = Raw4<T>::f(bv[i]);
    y[i] = make_float4(x.x + g.x * (acc.x + b.x), x.y + g.y * (acc.y + b.y), x.z + g.z * (acc.z + b.z),
                       x.w + g.w * (acc.w + b.w));
    *(float4*)(xr + 256 * i) = y[i];
    sum += (y[i].x + y[i].y) + (y[i].z + y[i].w);
  }
  const float mean = wave_sum_dpp(sum) / (float)d;
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const float a = y[i].x - mean, b = y[i].y - mean, e = y[i].z - mean, f = y[i].w - mean;
    sq += (a * a + b * b) + (e * e + f * f);
  }
  const float rstd = rsqrtf(wave_sum_dpp(sq) / (float)d + eps);
  T* hr = h + (size_t)row * d + 4 * lane;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const float4 sh = Raw4<float>::f(shv[i]), sc = Raw4<float>::f(scv[i]);
    Vec4Ld<T>::st(hr + 256 * i, make_float4((y[i].x - mean) * rstd * (1.0f + sc.x) + sh.x,
                                            (y[i].y - mean) * rstd * (1.0f + sc.y) + sh.y,
                                            (y[i].z - mean) * rstd * (1.0f + sc.z) + sh.z,
                                            (y[i].w - mean) * rstd * (1.0f + sc.w) + sh.w));
  }
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

struct TiledPlan {
  int cfg, nsplit;
};
static TiledPlan tiled_plan(int M, int N, int K);

size_t gemm_ws_floats(bool bf16, int M, int N, int K) {
  if (!bf16) return 0;
  if (use_skinny(M, K)) {
    SkinnyPlan p = skinny_plan(N, K);
    return p.nsplit > 1 ? (size_t)p.nsplit * M * N : 0;
  }
  const TiledPlan t = tiled_plan(M, N, K);
  return t.nsplit > 1 ? (size_t)t.nsplit * M * N : 0;
}

// Tile choice and K split for the tiled kernel: a function of (M, N, K)
// only, so one shape always runs one kernel and one reduction order.
// Shapes of the workloads take the configuration measured fastest for them
// on MI355X (sweep of the configurations and splits, event timing; the
// small-M shapes with the weights cold, as the model streams a new block's
// weights on every call -- warm L2 favours other tiles there); any
// other shape uses an estimate: the configuration's full-GPU rate (bf16
// TFLOP/s at M = 32768) x the fraction of its concurrent workgroup slots
// (256 CUs x workgroups per CU, set by LDS) its tiles keep busy over all
// rounds x the useful fraction of the (possibly ragged) tiles, and a K
// split when the tiles alone leave most CUs idle.
struct TileCfg {
  int bm, bn, per_cu;
  float rate;
};
// Two-stage tiles the size model chooses among (rate: sustained TFLOP/s
// measured on large square problems) ...
static const TileCfg kTiles[7] = {
    {256, 256, 1, 850.f}, {256, 192, 1, 800.f}, {128, 192, 2, 760.f}, {128, 128, 2, 740.f},
    {128, 96, 2, 700.f},  {64, 128, 3, 650.f},  {96, 128, 2, 600.f},
};
// ... and deeper-pipeline variants, chosen only by measurement:
// 7 = 128x96 with 4 stages, 8 = 96x128 with 3, 9 = 64x128 with 3, 10 = 128x128 with 3,
// and twelve-wavefront tiles (three per SIMD): 11 = 128x288 with 3 stages (2048 x 4608:
// exactly 256 tiles), 12 = 256x192 as 4 x 3 wavefronts of 64 x 64.
struct TileRule {
  int M, N, K, cfg, nsplit;
};
static const TileRule kMeasured[] = {
    // Fast-WAM scale video expert (2048 tokens): q|k|v in one launch, q|k, V^T, W_o, fc1, fc2
    {2048, 4608, 1536, 11, 1}, {2048, 3072, 1536, 4, 1}, {1536, 2048, 1536, 8, 1}, {2048, 1536, 1536, 7, 1},
    {2048, 6144, 1536, 12, 1}, {2048, 1536, 6144, 7, 1},
    // small model video expert (1024 tokens)
    {1024, 1536, 768, 5, 1}, {768, 1024, 768, 5, 1}, {1024, 768, 768, 5, 1}, {1024, 3072, 768, 4, 1},
    {1024, 768, 3072, 5, 1},
    // action expert over 512 rows (8 x 64 or 16 rollouts x 32 tokens) and 256 rows: q|k = fc1, V^T, W_o, fc2
    // (weights cold: each block streams its own)
    {512, 3072, 768, 9, 1}, {1536, 512, 768, 9, 1}, {512, 768, 1536, 9, 3}, {512, 768, 3072, 9, 4},
    {256, 3072, 768, 9, 1}, {256, 768, 3072, 9, 6},
    // video expert over 512 selected tokens (selective reuse): q|k, V^T, W_o, fc1, fc2 (weights cold)
    {512, 3072, 1536, 9, 1}, {1536, 512, 1536, 9, 2}, {512, 1536, 1536, 9, 2}, {512, 6144, 1536, 7, 1},
    {512, 1536, 6144, 7, 4},
};
static bool measured_shape(int M, int N, int K) {
  for (const TileRule& r : kMeasured)
    if (r.M == M && r.N == N && r.K == K) return true;
  return false;
}
static int pick_tile(int M, int N, int K) {
  int best = 3;
  float best_est = -1.f;
  for (int c = 0; c < 7; ++c) {
    const TileCfg& t = kTiles[c];
    const long tm = (M + t.bm - 1) / t.bm, tn = (N + t.bn - 1) / t.bn;
    const long tiles = tm * tn, slots = 256L * t.per_cu;
    const long rounds = (tiles + slots - 1) / slots;
    const float fill = (float)tiles / (float)(rounds * slots);
    const float useful = (float)M * (float)N / ((float)tiles * t.bm * t.bn);
    const float est = t.rate * fill * useful;
    if (est > best_est) {
      best_est = est;
      best = c;
    }
  }
  return best;
}

static TiledPlan tiled_plan(int M, int N, int K) {
  for (const TileRule& r : kMeasured)
    if (r.M == M && r.N == N && r.K == K) return {r.cfg, r.nsplit};
  TiledPlan p{pick_tile(M, N, K), 1};
  const TileCfg& t = kTiles[p.cfg < 7 ? p.cfg : 3];
  const long tiles = (long)((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
  // fewer tiles than half the CUs: split K (>= 4 K tiles per split, a
  // divisor of K / 64) until about 256 workgroups run
  if (N % 4 == 0 && tiles < 128) {
    const int kt = K / 64;
    for (int s = 2; s <= 16; ++s) {
      if (kt % s || kt / s < 4) continue;
      p.nsplit = s;
      if (tiles * s >= 256) break;
    }
  }
  return p;
}


// the weight-streaming kernel of plan p (partials into ws when it splits K)
template <class Epi>
static hipError_t skinny_main(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K, const Epi& epi,
                              const SkinnyPlan& p, float* ws, hipStream_t s) {
  dim3 grid(p.ntiles, p.nsplit);
  float* part = p.nsplit > 1 ? ws : nullptr;
  const bool w8 = p.chunks_per_split > 4;
  if (M <= 16) {
    if (w8) gemm_skinny_bf16<1, Epi, 8><<<grid, 512, 0, s>>>(A, lda, W, ldw, M, N, K, p.chunks_per_split, part, epi);
    else gemm_skinny_bf16<1, Epi><<<grid, 256, 0, s>>>(A, lda, W, ldw, M, N, K, p.chunks_per_split, part, epi);
  } else if (M <= 32) {
    if (w8) gemm_skinny_bf16<2, Epi, 8><<<grid, 512, 0, s>>>(A, lda, W, ldw, M, N, K, p.chunks_per_split, part, epi);
    else gemm_skinny_bf16<2, Epi><<<grid, 256, 0, s>>>(A, lda, W, ldw, M, N, K, p.chunks_per_split, part, epi);
  } else {
    if (w8) gemm_skinny_bf16<4, Epi, 8><<<grid, 512, 0, s>>>(A, lda, W, ldw, M, N, K, p.chunks_per_split, part, epi);
    else gemm_skinny_bf16<4, Epi><<<grid, 256, 0, s>>>(A, lda, W, ldw, M, N, K, p.chunks_per_split, part, epi);
  }
  return hipGetLastError();
}

bool gemm_gateres_ln_fusable(bool bf16, int M, int N, int K) {
  if (!bf16 || M < 1 || (N != 768 && N != 1536)) return false;
  if (use_skinny(M, K)) {
    const SkinnyPlan p = skinny_plan(N, K);
    return p.nsplit > 1 && p.nsplit <= 12;
  }
  if (K % 64) return false;
  const TiledPlan t = tiled_plan(M, N, K);
  return t.nsplit > 1 && t.nsplit <= 12;
}

// the K-split partials of the tiled kernel alone (plan p, nsplit > 1)
static hipError_t tiled_partials(const TiledPlan& p, const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N,
                                 int K, float* ws, hipStream_t s) {
  const EpiPart e{ws, N, (size_t)M * N};
  const int ns = p.nsplit;
  switch (p.cfg) {
    case 0: return run_tiled<256, 256, 2, 4, 2>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 1: return run_tiled<256, 192, 4, 2, 2>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 2: return run_tiled<128, 192, 2, 2, 2>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 3: return run_tiled<128, 128, 2, 2, 2>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 4: return run_tiled<128, 96, 4, 1, 2>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 5: return run_tiled<64, 128, 2, 2, 2>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 6: return run_tiled<96, 128, 1, 4, 2>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 7: return run_tiled<128, 96, 4, 1, 4>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 8: return run_tiled<96, 128, 1, 4, 3>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 9: return run_tiled<64, 128, 2, 2, 3>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 11: return run_tiled<128, 288, 4, 3, 3>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    case 12: return run_tiled<256, 192, 4, 3, 2>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
    default: return run_tiled<128, 128, 2, 2, 3>(A, lda, W, ldw, M, N, K, e, ns, ws, s);
  }
}

template <class T>
hipError_t launch_gemm_gateres_ln(const T* A, int lda, const T* W, int ldw, int M, int N, int K,
                                  const EpiGateRes<T>& epi, const float* shift, const float* scale, float eps, T* h,
                                  float* ws, hipStream_t s, int rows_per_group, size_t mod_stride) {
  if constexpr (sizeof(T) != 2) {
    return hipErrorInvalidValue;
  } else {
    if (!gemm_gateres_ln_fusable(true, M, N, K) || epi.ldx != N || !ws) return hipErrorInvalidValue;
    int nsplit;
    hipError_t e;
    if (use_skinny(M, K)) {
      const SkinnyPlan p = skinny_plan(N, K);
      nsplit = p.nsplit;
      e = skinny_main(A, lda, W, ldw, M, N, K, epi, p, ws, s);
    } else {
      const TiledPlan p = tiled_plan(M, N, K);
      nsplit = p.nsplit;
      e = tiled_partials(p, A, lda, W, ldw, M, N, K, ws, s);
    }
    if (e != hipSuccess) return e;
    const int grid = (M + 3) / 4;
#define WAM_FUSED(NCH, MAXS)                                                                                       \
  splitk_gateres_ln_kernel<T, NCH, MAXS><<<grid, 256, 0, s>>>(ws, nsplit, M, N, epi, shift, scale, eps, h,         \
                                                                 rows_per_group, mod_stride)
    if (N == 768) {
      if (nsplit <= 4) WAM_FUSED(3, 4);
      else if (nsplit <= 8) WAM_FUSED(3, 8);
      else WAM_FUSED(3, 12);
    } else {
      if (nsplit <= 4) WAM_FUSED(6, 4);
      else if (nsplit <= 8) WAM_FUSED(6, 8);
      else WAM_FUSED(6, 12);
    }
#undef WAM_FUSED
    return hipGetLastError();
  }
}
template hipError_t launch_gemm_gateres_ln<float>(const float*, int, const float*, int, int, int, int,
                                                  const EpiGateRes<float>&, const float*, const float*, float, float*,
                                                  float*, hipStream_t, int, size_t);
template hipError_t launch_gemm_gateres_ln<bf16_t>(const bf16_t*, int, const bf16_t*, int, int, int, int,
                                                   const EpiGateRes<bf16_t>&, const float*, const float*, float,
                                                   bf16_t*, float*, hipStream_t, int, size_t);

template <class Epi>
static hipError_t gemm_bf16(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K, const Epi& epi,
                            float* ws, hipStream_t s) {
  if (use_skinny(M, K)) {
    SkinnyPlan p = skinny_plan(N, K);
    hipError_t e = skinny_main(A, lda, W, ldw, M, N, K, epi, p, ws, s);
    if (e != hipSuccess || p.nsplit == 1) return e;
    gemm_splitk_reduce<Epi><<<(M * N + 255) / 256, 256, 0, s>>>(ws, p.nsplit, M, N, epi);
    return hipGetLastError();
  }
  if (K % 64) return hipErrorInvalidValue;
  const TiledPlan p = tiled_plan(M, N, K);
  const int ns = p.nsplit;
  // every configuration runs every epilogue without scratch (checked with
  // hipcc -Rpass-analysis=kernel-resource-usage), so the plan is used as is
  switch (p.cfg) {
    case 0: return run_tiled<256, 256, 2, 4, 2>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 1: return run_tiled<256, 192, 4, 2, 2>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 2: return run_tiled<128, 192, 2, 2, 2>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 3: return run_tiled<128, 128, 2, 2, 2>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 4: return run_tiled<128, 96, 4, 1, 2>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 5: return run_tiled<64, 128, 2, 2, 2>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 6: return run_tiled<96, 128, 1, 4, 2>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 7: return run_tiled<128, 96, 4, 1, 4>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 8: return run_tiled<96, 128, 1, 4, 3>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 9: return run_tiled<64, 128, 2, 2, 3>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 11: return run_tiled<128, 288, 4, 3, 3>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    case 12: return run_tiled<256, 192, 4, 3, 2>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
    default: return run_tiled<128, 128, 2, 2, 3>(A, lda, W, ldw, M, N, K, epi, ns, ws, s);
  }
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

size_t qkv_ws_floats(bool bf16, int M, int H, int dh, int K) {
  const int D = H * dh;
  size_t a = gemm_ws_floats(bf16, M, 3 * D, K);
  if (bf16 && !use_skinny(M, K)) a = std::max(gemm_ws_floats(bf16, M, 2 * D, K), gemm_ws_floats(bf16, D, M, K));
  return a;
}

template <class T>
hipError_t launch_qkv(const T* h, int M, int K, const T* W, const T* bias, int tokens, int H, int dh, T* q, T* k,
                      T* v, float* ws, hipStream_t s, const int* kv_tok, int kv_tokens) {
  const int D = H * dh;
  if (M <= 0) return hipSuccess;
  const bool two = sizeof(T) == 2 && !use_skinny(M, K);  // q|k, then V^T with swapped operands
  if (kv_tok) {
    const EpiQKVMap<T> eq{q, k, v, bias, M, H, dh, kv_tok, kv_tokens, fast_div(D), fast_div(dh)};
    if (!two) return launch_gemm<T>(h, K, W, K, M, 3 * D, K, eq, ws, s);
    hipError_t e = launch_gemm<T>(h, K, W, K, M, 2 * D, K, eq, ws, s);
    if (e != hipSuccess) return e;
    return launch_gemm<T>(W + (size_t)2 * D * K, K, h, K, D, M, K, EpiVTMap<T>{v, bias + 2 * D, kv_tokens, kv_tok},
                          ws, s);
  }
  const EpiQKV<T> eq{q, k, v, bias, tokens, H, dh, fast_div(D), fast_div(dh), fast_div(tokens)};
  if (!two) return launch_gemm<T>(h, K, W, K, M, 3 * D, K, eq, ws, s);
  // one launch where that was measured faster: the value columns go through
  // the epilogue's transposed stores (four tokens per 8-byte store)
  if (tokens % 4 == 0 && measured_shape(M, 3 * D, K)) return launch_gemm<T>(h, K, W, K, M, 3 * D, K, eq, ws, s);
  hipError_t e = launch_gemm<T>(h, K, W, K, M, 2 * D, K, eq, ws, s);
  if (e != hipSuccess) return e;
  return launch_gemm<T>(W + (size_t)2 * D * K, K, h, K, D, M, K, EpiVT<T>{v, bias + 2 * D, tokens, D, fast_div(tokens)}, ws, s);
}
template hipError_t launch_qkv<float>(const float*, int, int, const float*, const float*, int, int, int, float*,
                                      float*, float*, float*, hipStream_t, const int*, int);
template hipError_t launch_qkv<bf16_t>(const bf16_t*, int, int, const bf16_t*, const bf16_t*, int, int, int, bf16_t*,
                                       bf16_t*, bf16_t*, float*, hipStream_t, const int*, int);

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
