// Host-side launchers of the HIP kernels (one declaration per kernel
// family).  Every launcher enqueues on `s` and returns the launch status; it
// assumes its arguments were validated by the caller (wam_api.hip).
#pragma once

#include "common.h"

constexpr int WAM_MAX_T = 64;  // most flow times embedded by one launch

struct TList {
  float t[WAM_MAX_T];
  int n;
};

// E[j][k], j < ts.n: sinusoidal embedding of 1000 t_j, cosines then sines.
hipError_t launch_temb(const TList& ts, int dim, float* E, hipStream_t s);

// Y[j][n] = act_out(sum_k W[n][k] act_in(X[j][k]) + bias[n]),  j < J <= 16.
// W [N][K] in T, X [J][K] float32, Y [J][ldy] float32; act: 0 none, 1 SiLU.
// K must be a multiple of 8 and J*K <= 16384 (activations staged in 64 KB of LDS).
template <class T>
hipError_t launch_gemv(const T* W, int N, int K, const float* X, int J, int act_in,
                       const T* bias, int act_out, float* Y, int ldy, hipStream_t s);

// h[r][c] = LN(x[r])[c] (1 + scale[c]) + shift[c],  d a multiple of 4, d <= 8192.
template <class T>
hipError_t launch_ln_mod(const float* x, int rows, int d, const float* shift, const float* scale,
                         float eps, T* h, hipStream_t s, int rows_per_group = 1, size_t mod_stride = 0);

// x[i] = float(src[i]) for n elements.
template <class T>
hipError_t launch_to_f32(const T* src, size_t n, float* x, hipStream_t s);

// ---------------------------------------------------------------- selective reuse
// flags, then (in place) ascending indices of the tokens j with
// ||xn_j - xp_j||^2 > tau2 ||xp_j||^2 (float32 sums); count[0] = how many.
// idx holds T ints.
template <class T>
hipError_t launch_select_tokens(const T* xn, const T* xp, int T_tokens, int d, float tau2, int* idx, int* count,
                                hipStream_t s);
// x[r][:] = float(src[idx[r]][:]) for r < n
template <class T>
hipError_t launch_gather_rows(const T* src, const int* idx, int n, int d, float* x, hipStream_t s);
// dst[idx[r]][:] = x[r][:] for r < n
hipError_t launch_scatter_rows(const float* x, const int* idx, int n, int d, float* dst, hipStream_t s);
// QK-RMSNorm (gains g*, or NULL for none) + 3-D RoPE (rope_w > 0) on q and,
// if non-NULL, k: [B][H][Tn][dh] in place.
template <class T>
hipError_t launch_qk_norm_rope(T* q, const T* gq, T* k, const T* gk, int B, int H, int Tn, int dh, float eps,
                               int rope_h, int rope_w, hipStream_t s);

// y[m][n] = sum_k a[m][k] W[n][k] + b[n]; a float32 [M][A], W [d][A], y float32 [M][d].
template <class T>
hipError_t launch_action_in(const float* a, int M, int A, const T* W, const T* b, int d, float* y,
                            hipStream_t s);

// Final layer + Euler + endpoint, one row (action token) per workgroup:
//   v = (LN(y)(1+scale_f)+shift_f) W_out^T + b_out
//   a_next = a - dt v,  f = a - t v    (single fused multiply-adds)
// modf = [shift_f (d) | scale_f (d)].  a_next may alias a; v_out and f_out may be NULL.
template <class T>
hipError_t launch_final_euler(const float* y, int M, int d, const float* modf, const T* W_out,
                              const T* b_out, int A, float eps, const float* a, float dt, float t,
                              float* a_next, float* v_out, float* f_out, hipStream_t s, int rows_per_group = 1,
                              size_t mod_stride = 0, const TList* t_g = nullptr, const TList* dt_g = nullptr);
// Per-sample groups (rows_per_group > 0, mod_stride != 0 above): row group g
// takes its modulation at + g * mod_stride and its times t_g->t[g], dt_g->t[g].

// teacher-anchored targets over n = groups * per_group values (group g at time tg.t[g]):
// a_t = (1 - t) a0 + t eps (also into a_t_copy if non-NULL); u = (a_t - a) / t
hipError_t launch_targets_init(const float* a0, const float* eps, int n, int per_group, const TList& tg, float* a_t,
                               float* a_t_copy, hipStream_t s);
hipError_t launch_targets_u(const float* a_t, const float* a, int n, int per_group, const TList& tg, float* u,
                            hipStream_t s);

// ---------------------------------------------------------------- GEMM
// acc[m][n] = sum_k A[m][k] W[n][k]; each element goes to epi(m, n, acc).
// ws: float scratch of gemm_ws_floats(...) floats (split-K partial sums).
size_t gemm_ws_floats(bool bf16, int M, int N, int K);
template <class T, class Epi>
hipError_t launch_gemm(const T* A, int lda, const T* W, int ldw, int M, int N, int K, const Epi& epi,
                       float* ws, hipStream_t s);

// The gated-residual GEMM (x += gate (A W^T + bias)) whose K split's
// reduction also writes the next LayerNorm + modulation of the updated rows,
// h = LN(x)(1 + scale) + shift (per-sample modulation as launch_ln_mod).
// Only where gemm_gateres_ln_fusable(...) holds: bf16, N = 768 or 1536, and
// the shape's plan (weight-streaming for M <= 64, else tiled) splits K in
// 2..12; the result equals launch_gemm with EpiGateRes followed by
// launch_ln_mod.
bool gemm_gateres_ln_fusable(bool bf16, int M, int N, int K);
template <class T>
hipError_t launch_gemm_gateres_ln(const T* A, int lda, const T* W, int ldw, int M, int N, int K,
                                  const EpiGateRes<T>& epi, const float* shift, const float* scale, float eps, T* h,
                                  float* ws, hipStream_t s, int rows_per_group = 1, size_t mod_stride = 0);

// Merged q|k|v projection of M = B*tokens rows h [M][K] by W_qkv [3*H*dh][K]:
// q, k -> [B][H][tokens][dh], v -> [B][H][dh][tokens] (transposed).  With the
// tiled bf16 kernel this is one GEMM for the shapes measured faster that way
// (its epilogue stores the value columns four tokens at a time along V^T),
// otherwise two: q|k, then V^T = W_v h^T (operands swapped so the transposed
// result is written row-major).
// With kv_tok (one sample, M selected rows): q stays compact [H][M][dh]
// (tokens = M), k and v of row m go to token kv_tok[m] of a cache of
// kv_tokens tokens.
size_t qkv_ws_floats(bool bf16, int M, int H, int dh, int K);
template <class T>
hipError_t launch_qkv(const T* h, int M, int K, const T* W, const T* bias, int tokens, int H, int dh, T* q, T* k,
                      T* v, float* ws, hipStream_t s, const int* kv_tok = nullptr, int kv_tokens = 0);

// Debug hook: a kernel on `s` that just waits `us` microseconds (at most
// kMaxDebugDelayUs), so a test can make one stream late on purpose.
constexpr uint32_t kMaxDebugDelayUs = 10000;
hipError_t launch_delay(uint32_t us, hipStream_t s);

// ---------------------------------------------------------------- attention
// o[b][t][h*dh + e] = softmax over the keys [seg0 ; seg1] of q.k / sqrt(dh), times v.
// q [B][H][Tq][dh]; k0, v0 [B][H][L0][dh]; k1, v1 [B][H][L1][dh]; o [B][Tq][H*dh].
size_t attention_ws_floats(bool bf16, int B, int H, int dh, int Tq, int L0, int L1, int kv1_bcast = 0);
// A byte range (weights a later kernel of the same stream reads) that the
// bf16 attention (key-split instantiations) touches at its end: one 4-byte
// read per 128-byte line, which brings the range from HBM into the Infinity
// Cache, so the later kernel finds it there.  Results never depend on it.
struct AttnPrefetch {
  const void* p = nullptr;
  uint32_t bytes = 0u;  // 0, or >= 4 and a multiple of 4
};

template <class T>
hipError_t launch_attention(const T* q, const T* k0, const T* v0, int L0, const T* k1, const T* v1,
                            int L1, int B, int H, int dh, int Tq, T* o, float* ws, hipStream_t s,
                            int kv1_bcast = 0,  // kv1_bcast: segment 1 is one sample's, shared by all
                            const AttnPrefetch& pf = AttnPrefetch{});
