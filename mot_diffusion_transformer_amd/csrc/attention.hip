// Softmax attention over two concatenated key segments, the operation at the
// centre of the Mixture-of-Transformers coupling: the video expert attends
// over its own tokens (segment 1 empty); the action expert's block i
// attends over [own keys ; video block i keys].  No mask, scale 1/sqrt(dh).
//
// Keys are [B][H][L][dh]; values are stored TRANSPOSED, [B][H][dh][L], so the
// P.V product (a reduction over keys) reads keys contiguously.
//
// bf16 path: LDS-tiled online softmax on MFMA (attn_bf16_mfma below).  Long
// key ranges with few query tiles (the action expert: 32-64 queries against
// ~2-4k keys) are split over workgroups; the partial (max, sum, unnormalised
// output) triples are merged in split order by a second kernel.
//
// float32 path: one wavefront per query, online softmax over 64-key chunks.
#include "kernels.h"

#include <math.h>

#include <algorithm>

constexpr float kLog2e = 1.4426950408889634f;

template <class T>
WAM_DEV const T* key_row(const T* seg0, const T* seg1, int L0, int j, int dh) {
  return j < L0 ? seg0 + (size_t)j * dh : seg1 + (size_t)(j - L0) * dh;
}

// ============================================================================
// bf16 MFMA attention.
//
// Workgroup = QW wavefronts x 32 queries; a grid item is (sample x head,
// query tile, key split).  Per 64-key tile, each wavefront computes the
// transposed scores S^T = K Q^T on MFMA 32x32x16 (its 32 queries are the B
// operand, held in registers for the whole pass), so lane l ends up with 32
// scores of query l%32: keys 8(r/4) + 4(l/32) + r%4 of each 32-key half.
// After the online-softmax update those probabilities, rounded to bf16,
// are exactly the B operand of O^T += V^T P^T (k slots of lane half h in
// step ks: keys 16ks + 4h + {0..3} and 16ks + 8 + 4h + {0..3}), so P never
// leaves registers.  V is stored transposed ([dh][keys]) in the cache, so
// both operands come from LDS with plain 16/8-byte reads.
//
// K and V^T tiles are double-buffered in LDS and filled by direct
// global->LDS loads (XOR-swizzled 16-byte slots against bank conflicts);
// the next tile loads while the current one is consumed.  Tiles never
// straddle the two key segments; key rows past a segment's end read its
// last row and are masked out of the softmax, and V^T chunks that run past
// the end are assembled by the lanes themselves with zeros in the tail.
// ============================================================================
#define WAM_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

template <int VM>
WAM_DEV void wait_vm_lgkm0() {
  // s_waitcnt vmcnt(VM) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_waitcnt(0x0070 | (VM & 15) | ((VM >> 4) << 14));
}
WAM_DEV void block_barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int DH, int QW>
__global__ void __launch_bounds__(QW * 64, 2)
attn_bf16_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k0, const bf16_t* __restrict__ vt0, int L0,
               const bf16_t* __restrict__ k1, const bf16_t* __restrict__ vt1, int L1, int BH, int H, int Tq,
               int qtiles, int nsplit, int tiles_per_split, float scale_log2, bf16_t* __restrict__ o,
               float* __restrict__ part) {
  constexpr int KT = 64;                 // keys per tile
  constexpr int KCH = DH / 8;            // 16-byte chunks per K row
  constexpr int KROW = DH * 2;           // bytes per K row
  constexpr int VROW = KT * 2;           // bytes per V^T row (8 chunks)
  constexpr int K_BYTES = KT * KROW;
  constexpr int STAGE = K_BYTES + DH * VROW;
  constexpr int NCH = STAGE / 16;
  constexpr int LOADS = NCH / (64 * QW);
  static_assert(NCH % (64 * QW) == 0, "stage must split evenly over the wavefronts");
  static_assert(LOADS < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h32 = lane >> 5, l32 = lane & 31;

  // grid item: workgroups are dealt round-robin to the 8 XCDs; remap so each
  // XCD runs a contiguous range of (head, query tile) items and the head's
  // K/V stays in that XCD's L2
  const int items = BH * qtiles * nsplit;
  int id = blockIdx.x;
  if (items % 8 == 0) id = (id % 8) * (items / 8) + id / 8;
  const int sp = id % nsplit;
  const int rest = id / nsplit;
  const int qt = rest % qtiles;
  const int bh = rest / qtiles;
  const int b = bh / H, h = bh - b * H;

  const int nt0 = (L0 + KT - 1) / KT, nt1 = (L1 + KT - 1) / KT;
  const int t_beg = sp * tiles_per_split;
  const int t_end = min(nt0 + nt1, t_beg + tiles_per_split);
  const bf16_t* K0 = k0 + (size_t)bh * L0 * DH;
  const bf16_t* V0 = vt0 + (size_t)bh * DH * L0;
  const bf16_t* K1 = L1 > 0 ? k1 + (size_t)bh * L1 * DH : K0;
  const bf16_t* V1 = L1 > 0 ? vt1 + (size_t)bh * DH * L1 : V0;

  // this lane's query column and its fragments (B operand of S^T)
  const int qi = qt * 32 * QW + wave * 32 + l32;
  const bool qok = qi < Tq;
  bf16x8_t qf[DH / 16];
  {
    const bf16_t* qp = q + ((size_t)bh * Tq + (qok ? qi : 0)) * DH + h32 * 8;
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk) {
      uint4 u = qok ? *(const uint4*)(qp + kk * 16) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8_t, u);
    }
  }

  // Load slot P of a stage is a K chunk (row r, 16-byte chunk c of DH/8) or
  // a V^T chunk (row d, 8-key chunk c).  Each wave instruction covers 64
  // slots of one kind (K_LOADS instructions fill K), so the kind is uniform.
  constexpr int K_LOADS = (K_BYTES / 16) / 64;  // wave instructions that fill K
  // (row, element column) of load slot i, recomputed from the lane index (cheap, no registers held)
  auto slot_rc = [&](int i, int& row, int& col) {
    const int P = (wave * LOADS + i) * 64 + lane;
    if (P < K_BYTES / 16) {
      row = P / KCH;
      col = ((P % KCH) ^ (row & (KCH - 1))) * 8;
    } else {
      const int P2 = P - K_BYTES / 16;
      row = P2 >> 3;
      col = ((P2 & 7) ^ (row & 7)) * 8;
    }
  };
  // issue the direct loads of tile t into stage buffer `stg`
  auto issue = [&](int stg, int t) {
    const bool s0 = t < nt0;
    const int jt0 = (s0 ? t : t - nt0) * KT;
    const int Ls = s0 ? L0 : L1;
    const bf16_t* Kb = (s0 ? K0 : K1) + (size_t)jt0 * DH;
    const bf16_t* Vb = (s0 ? V0 : V1) + jt0;
    const bool full = jt0 + KT <= Ls;  // wave-uniform: no clamping or partial chunks
    unsigned char* base = smem + stg * STAGE + wave * LOADS * 1024;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      unsigned char* dst = base + i * 1024;  // this lane's slot is dst + lane * 16
      const bool is_k = (wave * LOADS + i) < K_LOADS;  // wave-uniform
      int lrow, lcol;
      slot_rc(i, lrow, lcol);
      if (is_k) {
        const int r = full ? lrow : min(lrow, Ls - jt0 - 1);
        __builtin_amdgcn_global_load_lds((const void*)(Kb + (size_t)r * DH + lcol), WAM_LDS_PTR(dst), 16, 0, 0);
      } else {
        const bf16_t* src = Vb + (size_t)lrow * Ls + lcol;
        if (full || jt0 + lcol + 8 <= Ls) {
          __builtin_amdgcn_global_load_lds((const void*)src, WAM_LDS_PTR(dst), 16, 0, 0);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          for (int e = 0; e < 8; ++e)
            if (jt0 + lcol + e < Ls) w[e >> 1] |= (uint32_t)src[e] << ((e & 1) * 16);
          *(uint4*)(dst + lane * 16) = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
  };

  f32x16_t oacc[DH / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  // m_ref: the exponent reference of this query's probabilities.  It only
  // moves (and O, l are rescaled) when a tile's max exceeds it by more than
  // RESCALE (log2 units), so probabilities stay below 2^RESCALE and the
  // rescale of the 64-float accumulator is rare.  The decision depends on
  // the data only, never on timing.
  constexpr float RESCALE = 8.0f;
  float m_ref = -INFINITY, l_run = 0.0f;

  if (t_beg < t_end) issue(0, t_beg);
  for (int t = t_beg; t < t_end; ++t) {
    // tile t is in LDS once this wave's loads for it are done (tile t+1 not yet issued)
    wait_vm_lgkm0<0>();
    block_barrier_nofence();
    if (t + 1 < t_end) issue((t + 1 - t_beg) & 1, t + 1);
    const unsigned char* st = smem + ((t - t_beg) & 1) * STAGE;
    const unsigned char* vs = st + K_BYTES;
    const bool s0 = t < nt0;
    const int valid = (s0 ? L0 : L1) - (s0 ? t : t - nt0) * KT;  // keys of this tile inside the segment

    f32x16_t s[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[ks][r] = 0.0f;
      const int row = ks * 32 + l32;
      const unsigned char* kp = st + row * KROW;
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        const int slot = ((2 * kk + h32) ^ (row & (KCH - 1))) * 16;
        s[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t*)(kp + slot), qf[kk], s[ks], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
    if (valid >= KT) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[ks][r] *= scale_log2;
          mx = fmaxf(mx, s[ks][r]);
        }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = ks * 32 + (r >> 2) * 8 + h32 * 4 + (r & 3);
          const float v = key < valid ? s[ks][r] * scale_log2 : -INFINITY;
          s[ks][r] = v;
          mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // finite: a tile holds >= 1 valid key
    if (__any(mx > m_ref + RESCALE)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DH / 32; ++i) oacc[i] *= alpha;
      m_ref = m_new;
    }
    float ls = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[ks][r] - m_ref);  // v_exp_f32; argument <= RESCALE
        s[ks][r] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32, 64);
    l_run += ls;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // P^T slots of step ks are registers 8(ks%2) .. 8(ks%2)+7 of half ks/2
      uint4 pu;
      const int r0 = (ks & 1) * 8;
      pu.x = pack_bf2(s[ks >> 1][r0 + 0], s[ks >> 1][r0 + 1]);
      pu.y = pack_bf2(s[ks >> 1][r0 + 2], s[ks >> 1][r0 + 3]);
      pu.z = pack_bf2(s[ks >> 1][r0 + 4], s[ks >> 1][r0 + 5]);
      pu.w = pack_bf2(s[ks >> 1][r0 + 6], s[ks >> 1][r0 + 7]);
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pu);
#pragma unroll
      for (int i = 0; i < DH / 32; ++i) {
        const int d = i * 32 + l32;
        const unsigned char* vr = vs + d * VROW + h32 * 8;
        const uint2 lo = *(const uint2*)(vr + (((2 * ks) ^ (d & 7)) * 16));
        const uint2 hi = *(const uint2*)(vr + (((2 * ks + 1) ^ (d & 7)) * 16));
        oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y)),
                                                          pf, oacc[i], 0, 0, 0);
      }
    }
  }
  const float m_run = m_ref;

  if (!qok) return;
  // O^T layout: register r of d-tile i holds d = 32i + 8(r/4) + 4h + r%4 of query l32
  if (nsplit == 1) {
    const float inv = 1.0f / l_run;
    bf16_t* op = o + ((size_t)b * Tq + qi) * (H * DH) + h * DH + h32 * 4;
#pragma unroll
    for (int i = 0; i < DH / 32; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 u;
        u.x = pack_bf2(oacc[i][4 * g] * inv, oacc[i][4 * g + 1] * inv);
        u.y = pack_bf2(oacc[i][4 * g + 2] * inv, oacc[i][4 * g + 3] * inv);
        *(uint2*)(op + i * 32 + g * 8) = u;
      }
  } else {
    // partial record [bh][split][query][DH + 4]: unnormalised o, then (m, l, -, -)
    float* pp = part + (((size_t)bh * nsplit + sp) * Tq + qi) * (DH + 4) + h32 * 4;
#pragma unroll
    for (int i = 0; i < DH / 32; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(pp + i * 32 + g * 8) = make_float4(oacc[i][4 * g], oacc[i][4 * g + 1], oacc[i][4 * g + 2], oacc[i][4 * g + 3]);
    if (h32 == 0) {
      float* pm = part + (((size_t)bh * nsplit + sp) * Tq + qi) * (DH + 4) + DH;
      pm[0] = m_run;
      pm[1] = l_run;
    }
  }
}

// Merge split partials in split order: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One wavefront per (sample x head, query); lane s holds split s's (m, l).
template <class T>
__global__ void __launch_bounds__(256)
attn_merge(const float* __restrict__ part, int nsplit, int BH, int H, int Tq, int dh, T* __restrict__ o) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= BH * Tq) return;
  const int bh = item / Tq, qi = item - bh * Tq;
  const int b = bh / H, h = bh - b * H;
  const size_t rec = (size_t)(dh + 4);
  const float* base = part + ((size_t)bh * nsplit * Tq + qi) * rec;
  const size_t sstride = (size_t)Tq * rec;
  float ms = -INFINITY, lsv = 0.0f;
  if (lane < nsplit) {
    ms = base[lane * sstride + dh];
    lsv = base[lane * sstride + dh + 1];
  }
  const float M = wave_max(ms);
  const float w = lane < nsplit ? exp2f(ms - M) : 0.0f;
  // fixed-order sum over splits (lane order), identical in every lane
  float l = 0.0f;
  for (int sp = 0; sp < nsplit; ++sp) l += __shfl(w, sp, 64) * __shfl(lsv, sp, 64);
  const float inv = 1.0f / l;
  for (int d = lane; d < dh; d += 64) {
    float acc = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) acc += __shfl(w, sp, 64) * base[sp * sstride + d];
    o[((size_t)b * Tq + qi) * (H * dh) + h * dh + d] = from_f32<T>(acc * inv);
  }
}

// ============================================================================
// float32 attention: one wavefront per query; 64-key chunks, lane j scores
// key j0 + j, then lanes own output features d = lane, lane + 64.  V is
// read transposed ([dh][keys]), as the bf16 path stores it.
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
  const float* V0 = v0 + (size_t)bh * dh * L0;  // V transposed: [dh][L0]
  const float* K1 = L1 > 0 ? k1 + (size_t)bh * L1 * dh : nullptr;
  const float* V1 = L1 > 0 ? v1 + (size_t)bh * dh * L1 : nullptr;
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
      const int j = j0 + jj;
      const float* vp = j < L0 ? V0 + j : V1 + (j - L0);  // column j of V^T
      const int ld = j < L0 ? L0 : L1;
      if (lane < dh) acc0 = fmaf(pj, vp[(size_t)lane * ld], acc0);
      if (lane + 64 < dh) acc1 = fmaf(pj, vp[(size_t)(lane + 64) * ld], acc1);
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
static AttnPlan attn_plan(int B, int H, int Tq, int L0, int L1) {
  AttnPlan p;
  p.qw = Tq <= 32 ? 1 : (Tq <= 64 ? 2 : 4);
  p.qtiles = (Tq + 32 * p.qw - 1) / (32 * p.qw);
  const int ntiles = (L0 + 63) / 64 + (L1 + 63) / 64;
  const int base = B * H * p.qtiles;
  // Many queries (video): a 4-wavefront item is efficient once the GPU is
  // full, so split keys only to reach ~1.5 items per CU (measured on MI355X:
  // 2048 tokens x 12 heads, 192 items -> 2 splits).  Few queries (action):
  // split the long key range into >= 4 parts and ~200 items (measured: 17
  // splits for 12 heads x 2080 keys, 4 for 96 sample-heads x 4160 keys).
  int want = p.qw == 4 ? (base >= 256 ? 1 : std::min(4, (384 + base - 1) / base))
                       : std::max(4, (200 + base - 1) / base);
  if (want > ntiles) want = ntiles;
  if (want < 1) want = 1;
  p.tiles_per_split = (ntiles + want - 1) / want;
  p.nsplit = (ntiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

size_t attention_ws_floats(bool bf16, int B, int H, int dh, int Tq, int L0, int L1) {
  if (!bf16) return 0;
  AttnPlan p = attn_plan(B, H, Tq, L0, L1);
  return p.nsplit > 1 ? (size_t)B * H * p.nsplit * Tq * (dh + 4) : 0;
}

template <int DH, int QW>
static void run_attn(const AttnPlan& p, const bf16_t* q, const bf16_t* k0, const bf16_t* v0, int L0, const bf16_t* k1,
                     const bf16_t* v1, int L1, int B, int H, int Tq, bf16_t* o, float* ws, hipStream_t s) {
  const int items = B * H * p.qtiles * p.nsplit;
  const float scale_log2 = kLog2e / sqrtf((float)DH);
  attn_bf16_mfma<DH, QW><<<items, QW * 64, 0, s>>>(q, k0, v0, L0, k1, v1, L1, B * H, H, Tq, p.qtiles, p.nsplit,
                                                    p.tiles_per_split, scale_log2, o, p.nsplit > 1 ? ws : nullptr);
}

template <int DH>
static void run_attn_dh(const AttnPlan& p, const bf16_t* q, const bf16_t* k0, const bf16_t* v0, int L0,
                        const bf16_t* k1, const bf16_t* v1, int L1, int B, int H, int Tq, bf16_t* o, float* ws,
                        hipStream_t s) {
  if (p.qw == 1) run_attn<DH, 1>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s);
  else if (p.qw == 2) run_attn<DH, 2>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s);
  else run_attn<DH, 4>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s);
}

template <class T>
hipError_t launch_attention(const T* q, const T* k0, const T* v0, int L0, const T* k1, const T* v1, int L1, int B,
                            int H, int dh, int Tq, T* o, float* ws, hipStream_t s) {
  if (Tq <= 0 || B <= 0) return hipSuccess;
  if (L0 + L1 <= 0) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2) {
    AttnPlan p = attn_plan(B, H, Tq, L0, L1);
    if (dh == 128) run_attn_dh<128>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s);
    else if (dh == 64) run_attn_dh<64>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s);
    else return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    attn_merge<bf16_t><<<(B * H * Tq + 3) / 4, 256, 0, s>>>(ws, p.nsplit, B * H, H, Tq, dh, o);
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
