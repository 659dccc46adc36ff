/*
 * wam_ops.h -- single-kernel entry points of the same library, for kernel
 * unit tests.  Each runs exactly the kernel (and launch-shape choice) that
 * the model uses for that operation, on caller-owned device buffers, and
 * enqueues on `stream` (a hipStream_t passed as void*).  Return WAM_OK or a
 * negative wam_status (see wam.h); nothing is enqueued on error.
 */
#ifndef WAM_OPS_H
#define WAM_OPS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogues of the model's linear layers (wam_op_gemm `epi`). */
typedef enum wam_epi {
  WAM_EPI_F32 = 0,      /* out float32 [M][N] = acc + bias                       */
  WAM_EPI_GELU = 1,     /* out dtype   [M][N] = GELU(acc + bias)  (MLP up)        */
  WAM_EPI_GATE_RES = 2, /* out float32 [M][N] += gate[n] (acc + bias)  (residual) */
  WAM_EPI_QKV = 3       /* out dtype: q, k [N/(3 dh)][M][dh] then v [N/(3 dh)][dh][M] */
} wam_epi;

/* acc[m][n] = sum_k A[m][k] W[n][k], then the epilogue `epi` (wam_epi).
 * A_dev [M][K], W_dev [N][K], bias_dev [N], all in `dtype` (wam_dtype);
 * gate_dev float32 [N] (WAM_EPI_GATE_RES only); head_dim (WAM_EPI_QKV only;
 * N must then be a multiple of 3*head_dim).  The model's y = x W^T + b
 * layers: merged q|k|v projection, output projection and MLP of each block.
 * Runs the same kernel instantiation and launch shape the model uses for
 * this (dtype, epi, M, N, K): the weight-streaming kernel for M <= 64 in
 * bf16, the tiled MFMA kernel otherwise.  K must be a multiple of 64 in
 * bf16; M, N >= 1.  ws_dev: wam_op_gemm_ws_bytes(dtype, M, N, K) bytes
 * (may be 0: split-K partial sums of the weight-streaming kernel).  Every
 * device pointer must be 16-byte aligned (the epilogues read and write up to
 * eight bf16 values in one access); otherwise WAM_ERR_ALIGN. */
size_t wam_op_gemm_ws_bytes(int dtype, int M, int N, int K);
int wam_op_gemm(int dtype, int epi, int M, int N, int K, const void* A_dev, const void* W_dev,
                const void* bias_dev, const float* gate_dev, int head_dim, void* out_dev, void* ws_dev,
                void* stream);

/* Multi-head softmax attention of queries over two concatenated key segments
 * (segment 0 then segment 1; either may be empty but not both), no mask,
 * scale 1/sqrt(dh):
 *   q_dev [B][H][Tq][dh]; k0 [B][H][L0][dh]; k1 [B][H][L1][dh]
 *   v0 [B][H][dh][L0], v1 [B][H][dh][L1]  (values transposed, as in the KV cache)
 *   o_dev [B][Tq][H*dh]
 * all in `dtype`.  The video expert's self-attention is L1 = 0; the action
 * expert's is segment 0 = its own keys, segment 1 = the video block's.
 * ws_dev: wam_op_attention_ws_bytes(...) bytes. */
size_t wam_op_attention_ws_bytes(int dtype, int B, int H, int dh, int Tq, int L0, int L1);
int wam_op_attention(int dtype, int B, int H, int dh, int Tq, const void* q_dev,
                     int L0, const void* k0_dev, const void* v0_dev,
                     int L1, const void* k1_dev, const void* v1_dev,
                     void* o_dev, void* ws_dev, void* stream);

/* h_dev[r][c] = ((x[r][c] - mean_r) / sqrt(var_r + eps)) (1 + scale[c]) + shift[c]
 * x_dev float32 [rows][d]; shift_dev, scale_dev float32 [d]; h_dev in dtype. */
int wam_op_ln_modulate(int dtype, int rows, int d, const float* x_dev, const float* shift_dev,
                       const float* scale_dev, float eps, void* h_dev, void* stream);

/* The block variant's fused QK-RMSNorm + 3-D RoPE on one q or k tensor, in
 * place (the operation wam.h describes under qk_norm / rope_height /
 * rope_width).  x_dev [B][H][T][dh] in dtype.  gain_dev [H*dh] in dtype, or
 * NULL for no normalisation; rope_height = rope_width = 0 for no rotation,
 * else T must be a multiple of rope_height*rope_width.  dh in {32, 64, 128}.
 * Returns WAM_ERR_SHAPE for sizes out of range, WAM_ERR_NULL for a NULL x. */
int wam_op_qk_norm_rope(int dtype, int B, int H, int T, int dh, void* x_dev, const void* gain_dev, float eps,
                        int rope_height, int rope_width, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WAM_OPS_H */
