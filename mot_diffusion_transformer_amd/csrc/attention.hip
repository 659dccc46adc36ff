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
// output) triples are merged in split order by a second kernel.  When every
// sample reads one shared segment 1 (rollouts of one observation), the
// workgroups over that segment take one sample per query wavefront, so each
// K/V tile is loaded once for several samples.
//
// float32 path: one wavefront per query, online softmax over 64-key chunks.
#include "kernels.h"

#include <math.h>

#include <algorithm>

constexpr float kLog2e = 1.4426950408889634f;
// Weight prefetch (below): one 4-byte read per 128-byte line brings the whole
// line in (measured: one read per 64 bytes gave fc2 the same speed-up); a
// wavefront read covers 64 lines.
constexpr uint32_t PF_LINE = 128u, PF_CHUNK = 64u * PF_LINE;

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
// scores of query l%32.  The K rows enter that product in a permuted order
// (below) chosen so that, after the online-softmax update, each lane's
// probabilities rounded to bf16 are exactly its B operand of
// O^T += V^T P^T for consecutive keys: P never leaves registers, and each
// V^T operand (V is stored transposed, [dh][keys], in the cache) is one
// 16-byte LDS read.
//
// K and V^T tiles are double-buffered in LDS and filled by direct
// global->LDS loads (XOR-swizzled 16-byte slots against bank conflicts);
// the next tile loads while the current one is consumed.  Tiles never
// straddle the two key segments; key rows past a segment's end read its
// last row and are masked out of the softmax, and V^T chunks that run past
// the end are assembled by the lanes themselves with zeros in the tail.
// ============================================================================

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

// Grid items: (sample x head, query tile, key split) or, with groups > 0
// (segment 1 shared by every sample, Tq <= 32), (head, group of QW
// samples, key split): query wavefront w then takes sample group*QW + w;
// there segment 0 (each sample's own L0 <= 64 keys) needs OWN, which adds
// it to split 0 from registers.  Results go out normalised when
// rec_nsplit == 1, otherwise as partial records at split rec_base + split
// of an array of rec_nsplit splits.
template <int DH, int QW, int KS, bool OWN = false>
__global__ void __launch_bounds__(QW * KS * 64, 2 / KS)
attn_bf16_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k0, const bf16_t* __restrict__ vt0, int L0,
               const bf16_t* __restrict__ k1, const bf16_t* __restrict__ vt1, int L1, int BH, int H, int Tq,
               int qtiles, int nsplit, int tiles_per_split, float scale_log2, bf16_t* __restrict__ o,
               float* __restrict__ part, int kv1_bcast, int groups, int rec_nsplit, int rec_base, AttnPrefetch pf) {
  constexpr int KT = 64;                 // keys per tile
  constexpr int KCH = DH / 8;            // 16-byte chunks per K row
  constexpr int KROW = DH * 2;           // bytes per K row
  constexpr int VROW = KT * 2;           // bytes per V^T row (8 chunks)
  constexpr int K_BYTES = KT * KROW;
  constexpr int STAGE = K_BYTES + DH * VROW;
  // KS key parts x 2 stages (dynamic: up to 128 KB)
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_all[];

  // KS > 1: the workgroup's key range is cut into KS parts, each run by its
  // own QW wavefronts (wave = kp * QW + query wave) over its own stages; the
  // parts' partial results meet in LDS at the end, so no partial record
  // leaves the chip.
  const int lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kp = wave_u / QW, wave = wave_u % QW;
  unsigned char* const smem = smem_all + kp * 2 * STAGE;
  const int h32 = lane >> 5, l32 = lane & 31;

  // grid item: workgroups are dealt round-robin to the 8 XCDs; remap so each
  // XCD runs a contiguous range of (head, query tile) items and the head's
  // K/V stays in that XCD's L2
  const int items = (groups > 0 ? H * groups : BH * qtiles) * nsplit;
  int id = blockIdx.x;
  if (items % 8 == 0) id = (id % 8) * (items / 8) + id / 8;
  const int sp = id % nsplit;
  const int rest = id / nsplit;
  int qt, b, h;
  if (groups > 0) {
    qt = 0;
    h = rest / groups;
    b = (rest - h * groups) * QW + wave;  // past the last sample: loads and barriers only
  } else {
    qt = rest % qtiles;
    b = rest / qtiles / H;
    h = rest / qtiles - b * H;
  }
  const int bh = b * H + h;

  // OWN (groups > 0): every sample's own keys (L0 <= 64) are not tiles but a
  // register prologue of split 0 (below)
  const bool own = OWN && groups > 0 && L0 > 0;
  const int nt0 = own ? 0 : (L0 + KT - 1) / KT, nt1 = (L1 + KT - 1) / KT;
  const int w_beg = sp * tiles_per_split;
  const int w_end = min(nt0 + nt1, w_beg + tiles_per_split);
  // this part's tiles; every part runs `iters` iterations (barriers are shared)
  const int iters = (w_end - w_beg + KS - 1) / KS;
  const int t_beg = min(w_end, w_beg + kp * iters);
  const int t_end = min(w_end, t_beg + iters);
  const bf16_t* K0 = k0 + (size_t)bh * L0 * DH;
  const bf16_t* V0 = vt0 + (size_t)bh * DH * L0;
  // segment 1 shared by every sample (kv1_bcast): indexed by head only
  const int bh1 = kv1_bcast ? h : bh;
  const bf16_t* K1 = L1 > 0 ? k1 + (size_t)bh1 * L1 * DH : K0;
  const bf16_t* V1 = L1 > 0 ? vt1 + (size_t)bh1 * DH * L1 : V0;

  // this lane's query column and its fragments (B operand of S^T)
  const int qi = groups > 0 ? l32 : qt * 32 * QW + wave * 32 + l32;
  const bool qok = qi < Tq && bh < BH;
  bf16x8_t qf[DH / 16];
  {
    // Loads here and below are unconditional, from clamped addresses, with
    // the zeros put in afterwards: a load under a per-lane condition whose
    // other lanes get a constant makes the compiler wait for that load before
    // the next one, one memory round trip each.
    const bf16_t* qp = q + (qok ? (size_t)bh * Tq + qi : 0) * DH + h32 * 8;
    uint4 qu[DH / 16];
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk) qu[kk] = *(const uint4*)(qp + kk * 16);
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8_t, qok ? qu[kk] : make_uint4(0, 0, 0, 0));
  }

  // Stage layout: K tile [64 keys][DH] then V^T tile [DH][64 keys], both in
  // 16-byte chunks XOR-swizzled per row (K: chunk ^ (row % KCH), V^T: chunk ^
  // (row % 8)).  Each wavefront fills KL wave-instructions of K and VL of V^T
  // (1 KB each: 64 lanes x 16 B), so the kind of every load is static.
  constexpr int KL = K_BYTES / 1024 / QW, VL = (STAGE - K_BYTES) / 1024 / QW;
  static_assert(KL * QW * 1024 == K_BYTES && VL * QW * 1024 == STAGE - K_BYTES, "loads split evenly");
  // Tiles arrive by buffer_load ... lds (MUBUF: unlike a FLAT load into LDS
  // it lets the compiler wait for LDS reads one at a time).  Descriptors span
  // this (sample, head)'s K and V^T of each segment; the tile's first key
  // goes in the scalar offset.
  const BufRsrc rk0 = buf_rsrc(K0, (uint32_t)L0 * DH * 2), rv0 = buf_rsrc(V0, (uint32_t)L0 * DH * 2);
  const BufRsrc rk1 = buf_rsrc(K1, (uint32_t)L1 * DH * 2), rv1 = buf_rsrc(V1, (uint32_t)L1 * DH * 2);
  // issue the direct loads of tile t into stage buffer `stg`
  auto issue = [&](int stg, int t) {
    const bool s0 = t < nt0;
    const int jt0 = (s0 ? t : t - nt0) * KT;
    const int Ls = s0 ? L0 : L1;
    const bool full = jt0 + KT <= Ls;  // uniform
    unsigned char* kbase = smem + stg * STAGE + wave * KL * 1024;
    unsigned char* vbase = smem + stg * STAGE + K_BYTES + wave * VL * 1024;
    // slot arithmetic is redone per tile (a few integer ops): hoisted out of
    // the tile loop it would pin one address register per load
    uint32_t ln = lane;
    asm volatile("" : "+v"(ln));
    constexpr uint32_t KSH = DH == 128 ? 4 : 3;  // log2(KCH)
    static_assert((1 << KSH) == KCH, "K chunks per row");
#pragma unroll
    for (int j = 0; j < KL; ++j) {
      const uint32_t P = (uint32_t)(wave * KL + j) * 64u + ln;
      const uint32_t row = P >> KSH, col = ((P ^ row) & (KCH - 1)) * 8;
      const uint32_t r = full ? row : min(row, (uint32_t)(Ls - jt0 - 1));  // rows past the end repeat the last
      buf_load_lds16(s0 ? rk0 : rk1, kbase + j * 1024, (r * DH + col) * 2, (uint32_t)jt0 * DH * 2);
    }
    // A whole tile (uniform) takes straight-line loads: the per-chunk test
    // below would put a branch around every one of them.
    if (full) {
#pragma unroll
      for (int j = 0; j < VL; ++j) {
        const uint32_t P = (uint32_t)(wave * VL + j) * 64u + ln;
        const uint32_t d = P >> 3, col = ((P ^ d) & 7) * 8;
        buf_load_lds16(s0 ? rv0 : rv1, vbase + j * 1024, (d * (uint32_t)Ls + col) * 2, (uint32_t)jt0 * 2);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < VL; ++j) {
      const uint32_t P = (uint32_t)(wave * VL + j) * 64u + ln;
      const uint32_t d = P >> 3, col = ((P ^ d) & 7) * 8;
      if (jt0 + (int)col + 8 <= Ls) {
        buf_load_lds16(s0 ? rv0 : rv1, vbase + j * 1024, (d * (uint32_t)Ls + col) * 2, (uint32_t)jt0 * 2);
      } else {
        // the chunk runs past the segment's end: zeros, and where it starts
        // inside (a length that is not a multiple of 8) assembled by hand
        // from reads clamped to the row's last key
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (jt0 + (int)col < Ls) {
          const bf16_t* vrow = (s0 ? V0 : V1) + (size_t)d * Ls;
          uint32_t x[8], w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = vrow[min(jt0 + (int)col + e, Ls - 1)];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (jt0 + (int)col + e < Ls) w[e >> 1] |= x[e] << ((e & 1) * 16);
          val = make_uint4(w[0], w[1], w[2], w[3]);
        }
        *(uint4*)(vbase + j * 1024 + lane * 16) = val;
      }
    }
  };

  // Key order.  Row i (0..31) of each 32-key half of the S^T MFMA's A
  // operand holds key pi(i) of that half, pi swapping bits 2 and 3 of i.
  // Output register r of lane half h is row 8(r/4) + 4h + r%4, so it holds
  // key 16(g/2) + 8h + 4(g%2) + r%4 (g = r/4): registers 8j..8j+7 of half
  // hh are keys 32hh + 16j + 8h + 0..7, in order.  Those eight
  // probabilities are exactly lane half h's k-slots (8h..8h+7) of P.V step
  // 2hh + j with key = 16 step + slot, so the matching V^T operand is the
  // 16-byte chunk 2 step + h of row d: one LDS read.
  const int pil = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  // Per-lane LDS read offsets within a stage: K fragment kk of half 0 (half
  // 1 is 32 rows on, same swizzle key: an immediate), V^T fragment of step ks
  // for d-tile 0 (d-tiles are immediates apart too).
  int koff[DH / 16], voff[4];
#pragma unroll
  for (int kk = 0; kk < DH / 16; ++kk) koff[kk] = pil * KROW + (((2 * kk + h32) ^ (pil & (KCH - 1))) * 16);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) voff[ks] = K_BYTES + l32 * VROW + (((2 * ks + h32) ^ (l32 & 7)) * 16);

  f32x16_t oacc[DH / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  // m_ref: the exponent reference of this query's probabilities (log2
  // units, scale applied).  It only moves (and O, l are rescaled) when a
  // tile's max exceeds it by more than RESCALE, so probabilities stay below
  // 2^RESCALE and the rescale of the accumulator is rare.  The decision
  // depends on the data only, never on timing.
  constexpr float RESCALE = 8.0f;
  float m_ref = -INFINITY, l_run = 0.0f;

  // The sample's own L0 (<= 64) keys, first and only in split 0 (key part
  // 0), as one partial tile whose fragments come straight from memory in
  // the MFMA operand order of the tile loop below (K row 32 half + pil,
  // chunk 2 kk + h32; V^T row d, keys 16 step + 8 h32 ..), zeros past the
  // last key.  The arithmetic is the tile loop's, written out again so that
  // the kernels without this prologue keep their register allocation.
  if constexpr (OWN) {
    if (own && sp == 0 && kp == 0 && bh < BH) {
      // a 32-key half with no key at all (ks 32 >= L0, uniform) is not read
      bf16x8_t kf[2][DH / 16];
      uint4 ku[2][DH / 16];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int key = min(ks * 32 + pil, L0 - 1);
#pragma unroll
        for (int kk = 0; kk < DH / 16; ++kk)
          ku[ks][kk] = ks * 32 < L0 ? *(const uint4*)(K0 + (size_t)key * DH + (2 * kk + h32) * 8) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int kk = 0; kk < DH / 16; ++kk)
          kf[ks][kk] = __builtin_bit_cast(bf16x8_t, ks * 32 + pil < L0 ? ku[ks][kk] : make_uint4(0, 0, 0, 0));
      f32x16_t s[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[ks][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) s[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks][kk], qf[kk], s[ks], 0, 0, 0);
      bf16x8_t vf[4][DH / 32];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < DH / 32; ++i) {
          const int key0 = ks * 16 + h32 * 8;
          const bf16_t* vrow = V0 + (size_t)(l32 + 32 * i) * L0;
          uint32_t wv[4] = {0u, 0u, 0u, 0u};
          if (ks * 16 < L0) {  // uniform: this 16-key step has keys
            if (L0 % 8 == 0) {  // whole 16-byte chunks: one read, clamped to the last chunk
              const uint4 u = *(const uint4*)(vrow + min(key0, L0 - 8));
              if (key0 < L0) wv[0] = u.x, wv[1] = u.y, wv[2] = u.z, wv[3] = u.w;
            } else {
              uint32_t x[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) x[e] = vrow[min(key0 + e, L0 - 1)];
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (key0 + e < L0) wv[e >> 1] |= x[e] << ((e & 1) * 16);
            }
          }
          vf[ks][i] = __builtin_bit_cast(bf16x8_t, make_uint4(wv[0], wv[1], wv[2], wv[3]));
        }
      // first keys of this query: the reference is the (masked) max itself
      float mx = -INFINITY;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int g = r >> 2;
          const int key = ks * 32 + (g >> 1) * 16 + h32 * 8 + (g & 1) * 4 + (r & 3);
          if (key >= L0) s[ks][r] = -INFINITY;
          mx = fmaxf(mx, s[ks][r]);
        }
      m_ref = halves_max(mx) * scale_log2;  // finite: L0 >= 1
      float ls = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ks][r], scale_log2, -m_ref));
          s[ks][r] = p;
          ls += p;
        }
      l_run = halves_sum(ls);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        uint4 pu;
        const int r0 = (ks & 1) * 8;
        pu.x = pack_bf2(s[ks >> 1][r0 + 0], s[ks >> 1][r0 + 1]);
        pu.y = pack_bf2(s[ks >> 1][r0 + 2], s[ks >> 1][r0 + 3]);
        pu.z = pack_bf2(s[ks >> 1][r0 + 4], s[ks >> 1][r0 + 5]);
        pu.w = pack_bf2(s[ks >> 1][r0 + 6], s[ks >> 1][r0 + 7]);
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pu);
#pragma unroll
        for (int i = 0; i < DH / 32; ++i) oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks][i], pf, oacc[i], 0, 0, 0);
      }
    }
  }

  // Weight prefetch (KS == 2 only, whose end waits for every load before
  // the merge): PF 4-byte DMA reads per wavefront into a 256-byte LDS sink
  // past the stages, lane l at byte l PF_LINE of a PF_CHUNK chunk (PF = 2
  // covers 25 MB at 192 workgroups of 8 wavefronts); chunk c goes to
  // wavefront c % NW of workgroup (c / NW) % gridDim.x, so neighbouring
  // chunks are read by different CUs.  They are issued once every tile of
  // the workgroup is in (the last iteration), and their HBM round trip runs
  // under the last tile's products: issued while tile loads were still to
  // come, they held those up (a CU's loads return in order).  Wavefronts
  // whose chunks lie past the range read nothing; every offset is clamped
  // inside the range.
  constexpr int PF = 2;
  const bool pf_on = KS == 2 && pf.bytes != 0u;  // uniform
  auto prefetch = [&]() {
    constexpr uint32_t NW = QW * KS;
    const uint32_t nchunk = (pf.bytes + PF_CHUNK - 1u) / PF_CHUNK;
    const BufRsrc r = buf_rsrc(pf.p, pf.bytes);
    unsigned char* sink = smem_all + KS * 2 * STAGE + wave_u * 256;
#pragma unroll
    for (uint32_t j = 0; j < PF; ++j) {
      const uint32_t c = (j * gridDim.x + blockIdx.x) * NW + wave_u;  // uniform
      if (c >= nchunk) break;  // past the range: nothing to read (with more workgroups than chunks)
      const uint32_t off = min(c * PF_CHUNK + (uint32_t)lane * PF_LINE, pf.bytes - 4u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, WAM_LDS_PTR(sink), 4, off, 0, 0, 0);
    }
  };

  if (t_beg < t_end) issue(0, t_beg);
  for (int it = 0; it < iters; ++it) {
    const int t = t_beg + it;
    // tile t is in LDS once this wave's loads for it are done (tile t+1 not yet issued)
    wait_vm_lgkm0<0>();
    block_barrier_nofence();
    if (t >= t_end) continue;  // a shorter part idles through the remaining barriers
    if (t + 1 < t_end) issue((t + 1 - t_beg) & 1, t + 1);
    else if (pf_on) prefetch();
    const unsigned char* st = smem + ((t - t_beg) & 1) * STAGE;
    const bool s0 = t < nt0;
    const int valid = (s0 ? L0 : L1) - (s0 ? t : t - nt0) * KT;  // keys of this tile inside the segment

    // S^T = K Q^T for the two 32-key halves: every K fragment of the tile is
    // read first, then the two independent MFMA chains run interleaved, each
    // step waiting only for its own fragment (the scheduling groups keep the
    // compiler from sinking each read next to its MFMA).
    bf16x8_t kf[2][DH / 16];
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk) {
      const unsigned char* kp = st + koff[kk];
      kf[0][kk] = *(const bf16x8_t*)kp;
      kf[1][kk] = *(const bf16x8_t*)(kp + 32 * KROW);
    }
    f32x16_t s[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[ks][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) s[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks][kk], qf[kk], s[ks], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, DH / 8, 0);  // the K fragment reads
    __builtin_amdgcn_sched_group_barrier(0x008, DH / 8, 0);  // then the S MFMAs
    __builtin_amdgcn_sched_barrier(0);  // the V^T fragments below reuse the K fragments' registers
    // V^T fragments of the whole tile (B operand order of O^T += V^T P^T),
    // read before the softmax so their latency hides under it
    bf16x8_t vf[4][DH / 32];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < DH / 32; ++i) vf[ks][i] = *(const bf16x8_t*)(st + voff[ks] + i * 32 * VROW);
    __builtin_amdgcn_sched_barrier(0);

    // softmax statistics on the raw scores (the scale is positive, so the
    // max commutes with it); probabilities as exp2(s * scale - m_ref)
    float mx = -INFINITY;
    if (valid < KT) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int g = r >> 2;
          const int key = ks * 32 + (g >> 1) * 16 + h32 * 8 + (g & 1) * 4 + (r & 3);
          if (key >= valid) s[ks][r] = -INFINITY;
        }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[ks][r]);
    mx = halves_max(mx) * scale_log2;  // finite: a tile holds >= 1 valid key
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
        // v_exp_f32; the argument is <= RESCALE
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ks][r], scale_log2, -m_ref));
        s[ks][r] = p;
        ls += p;
      }
    ls = halves_sum(ls);
    l_run += ls;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // P^T slots of step ks are registers 8(ks%2) .. 8(ks%2)+7 of half ks/2 (key order above)
      uint4 pu;
      const int r0 = (ks & 1) * 8;
      pu.x = pack_bf2(s[ks >> 1][r0 + 0], s[ks >> 1][r0 + 1]);
      pu.y = pack_bf2(s[ks >> 1][r0 + 2], s[ks >> 1][r0 + 3]);
      pu.z = pack_bf2(s[ks >> 1][r0 + 4], s[ks >> 1][r0 + 5]);
      pu.w = pack_bf2(s[ks >> 1][r0 + 6], s[ks >> 1][r0 + 7]);
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pu);
#pragma unroll
      for (int i = 0; i < DH / 32; ++i) oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks][i], pf, oacc[i], 0, 0, 0);
    }
  }
  float m_run = m_ref;
  if constexpr (KS == 2) {
    // part 1 parks (m, l, O^T) in the freed stage buffers; part 0's lane of
    // the same query wave holds the same (query, feature) elements and merges
    // them in fixed order
    constexpr int REC = DH / 32 * 16 + 4;  // floats per lane
    static_assert(QW * 64 * REC * 4 <= KS * 2 * STAGE, "merge records fit in the stages");
    float* rec = (float*)smem_all + ((size_t)wave * 64 + lane) * REC;
    wait_vm_lgkm0<0>();
    block_barrier_nofence();  // every part is done with its stages
    if (kp == 1) {
#pragma unroll
      for (int i = 0; i < DH / 32; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(float4*)(rec + i * 16 + g * 4) = make_float4(oacc[i][4 * g], oacc[i][4 * g + 1], oacc[i][4 * g + 2], oacc[i][4 * g + 3]);
      *(float2*)(rec + DH / 32 * 16) = make_float2(m_ref, l_run);
    }
    wait_vm_lgkm0<0>();
    block_barrier_nofence();
    if (kp == 1) return;
    const float2 ml = *(const float2*)(rec + DH / 32 * 16);
    const float m_new = fmaxf(m_ref, ml.x);  // finite: the workgroup saw >= 1 key
    const float w0 = __builtin_amdgcn_exp2f(m_ref - m_new), w1 = __builtin_amdgcn_exp2f(ml.x - m_new);
    l_run = w0 * l_run + w1 * ml.y;
#pragma unroll
    for (int i = 0; i < DH / 32; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 o1 = *(const float4*)(rec + i * 16 + g * 4);
        oacc[i][4 * g] = w0 * oacc[i][4 * g] + w1 * o1.x;
        oacc[i][4 * g + 1] = w0 * oacc[i][4 * g + 1] + w1 * o1.y;
        oacc[i][4 * g + 2] = w0 * oacc[i][4 * g + 2] + w1 * o1.z;
        oacc[i][4 * g + 3] = w0 * oacc[i][4 * g + 3] + w1 * o1.w;
      }
    m_run = m_new;
  }

  if (!qok) return;
  // O^T layout: register r of d-tile i holds d = 32i + 8(r/4) + 4h + r%4 of query l32
  if (rec_nsplit == 1) {
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
    const size_t rec = ((size_t)bh * rec_nsplit + rec_base + sp) * Tq + qi;
    float* pp = part + rec * (DH + 4) + h32 * 4;
#pragma unroll
    for (int i = 0; i < DH / 32; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(pp + i * 32 + g * 8) = make_float4(oacc[i][4 * g], oacc[i][4 * g + 1], oacc[i][4 * g + 2], oacc[i][4 * g + 3]);
    if (h32 == 0) {
      float* pm = part + rec * (DH + 4) + DH;
      pm[0] = m_run;
      pm[1] = l_run;
    }
  }
}

// Merge split partials in split order: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One wavefront per (sample x head, query); lane l owns features 2l, 2l+1
// (dh <= 128).  Every lane reads every split's (m, l) itself (the same
// addresses in all lanes) and forms the weights 2^(m_s - M) on its own, so no
// value crosses lanes; SB (4, 8 or 16: the split count rounded up) splits'
// statistics and output rows are requested at once, unconditionally from
// clamped positions (a guarded load would be waited for at its branch),
// before any is used.  M is the exact maximum and the sums run in split
// order.
template <class T, int SB>
__global__ void __launch_bounds__(256)
attn_merge(const float* __restrict__ part, int nsplit, int BH, int H, int Tq, int dh, T* __restrict__ o) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= BH * Tq) return;  // uniform per wavefront
  const int bh = item / Tq, qi = item - bh * Tq;
  const int b = bh / H, h = bh - b * H;
  const size_t rec = (size_t)(dh + 4);
  const float* base = part + ((size_t)bh * nsplit * Tq + qi) * rec;
  const size_t sstride = (size_t)Tq * rec;
  const int d = 2 * lane;
  const bool dok = d < dh;
  const int dc = dok ? d : 0;  // lanes past dh read (and drop) the first pair
  float M = -INFINITY;
  if (nsplit > SB) {  // uniform: the maximum first, over every split
    for (int s0 = 0; s0 < nsplit; s0 += SB) {
      float mv[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j) mv[j] = base[(size_t)min(s0 + j, nsplit - 1) * sstride + dh];
#pragma unroll
      for (int j = 0; j < SB; ++j) M = fmaxf(M, mv[j]);  // repeats of the last split change nothing
    }
  }
  float l = 0.0f, ax = 0.0f, ay = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += SB) {
    float mv[SB], lv[SB];
    float2 v[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const float* pj = base + (size_t)min(s0 + j, nsplit - 1) * sstride;
      mv[j] = pj[dh];
      lv[j] = pj[dh + 1];
      v[j] = *(const float2*)(pj + dc);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above is in flight before the first use
    if (nsplit <= SB) {
#pragma unroll
      for (int j = 0; j < SB; ++j) M = fmaxf(M, mv[j]);
    }
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      if (s0 + j < nsplit) {  // uniform
        const float w = exp2f(mv[j] - M);
        l += w * lv[j];
        ax += w * v[j].x;
        ay += w * v[j].y;
      }
    }
  }
  const float inv = 1.0f / l;
  if (dok) {
    T* op = o + ((size_t)b * Tq + qi) * (H * dh) + h * dh + d;
    op[0] = from_f32<T>(ax * inv);
    op[1] = from_f32<T>(ay * inv);
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
         float* __restrict__ o, int kv1_bcast) {
  const int lane = threadIdx.x & 63;
  const int qi = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int bh = blockIdx.y;
  if (qi >= Tq) return;
  const int b = bh / H, h = bh - b * H;
  const int L = L0 + L1;
  const float* K0 = k0 + (size_t)bh * L0 * dh;
  const float* V0 = v0 + (size_t)bh * dh * L0;  // V transposed: [dh][L0]
  const int bh1 = kv1_bcast ? h : bh;  // segment 1 shared by every sample
  const float* K1 = L1 > 0 ? k1 + (size_t)bh1 * L1 * dh : nullptr;
  const float* V1 = L1 > 0 ? v1 + (size_t)bh1 * dh * L1 : nullptr;
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
  int qw, ks, qtiles, nsplit, tiles_per_split;
};
static AttnPlan attn_plan(int B, int H, int Tq, int L0, int L1) {
  AttnPlan p;
  p.qw = Tq <= 32 ? 1 : (Tq <= 64 ? 2 : 4);
  p.qtiles = (Tq + 32 * p.qw - 1) / (32 * p.qw);
  const int ntiles = (L0 + 63) / 64 + (L1 + 63) / 64;
  const int base = B * H * p.qtiles;
  // Many queries (video): 4 query wavefronts per item.  Under ~256 items
  // (2048 tokens x 12 heads: 192) the keys are cut in two inside the
  // workgroup (8 wavefronts, merged in LDS), which fills the SIMDs without
  // a partial record through memory; with more items the GPU is full as it
  // is.  Few queries (action): split the long key range over workgroups into
  // >= 4 parts and ~132 items (measured on MI355X: 11 splits for 12 heads x
  // 2080 keys, 4 for 96 sample-heads x 4160 keys), merged by a second kernel.
  // Few query items even with the key halves (under 64: e.g. a few hundred
  // selected queries of one sample): the keys are also split over
  // workgroups, up to ~256 workgroups and >= 4 key tiles per split.
  int want = 1;
  p.ks = 1;
  if (p.qw == 4) {
    if (base < 256 && ntiles >= 2) p.ks = 2;
    if (p.ks == 2 && base < 64) want = std::max(1, std::min(ntiles / 4, 256 / base));
  } else {
    want = std::max(4, (132 + base - 1) / base);
  }
  if (want > ntiles) want = ntiles;
  if (want > 64) want = 64;  // at most 64 splits (partial records: 64 x (dh + 4) floats per query)
  if (want < 1) want = 1;
  p.tiles_per_split = (ntiles + want - 1) / want;
  p.nsplit = (ntiles + p.tiles_per_split - 1) / p.tiles_per_split;
  // one query wavefront: its split's tiles are also cut in two inside the
  // workgroup (2 wavefronts), so two key tiles load at once (32 queries over
  // 2080 keys x 12 heads: 19.4 -> 17.3 us with the merge, measured on MI355X)
  if (p.qw == 1 && p.tiles_per_split >= 2) p.ks = 2;
  return p;
}

// Shared segment 1 (kv1_bcast) with several samples of <= 32 queries:
// segment 1 runs as (head, group of 4 samples, key split) workgroups of
// 2 x 4 wavefronts (keys cut in two inside the workgroup), at most one per
// CU, with >= 2 key tiles per split; each sample's own keys (<= 64) are
// folded into split 0 from registers; all splits merge in order.
struct GroupPlan {
  int groups, nsplit, tiles_per_split, rec;
};
// (the own keys, at most one 64-key tile, are read into registers)
static bool use_groups(int B, int Tq, int L0, int L1, int kv1_bcast) {
  return kv1_bcast && B > 1 && L1 > 0 && Tq <= 32 && L0 <= 64;
}
static GroupPlan group_plan(int B, int H, int L0, int L1) {
  GroupPlan g;
  g.groups = (B + 3) / 4;
  const int nt1 = (L1 + 63) / 64;
  int want = std::max(1, 256 / (H * g.groups));
  want = std::min(want, std::max(1, nt1 / 2));
  want = std::min(want, 64);  // at most 64 splits, as above
  g.tiles_per_split = (nt1 + want - 1) / want;
  g.nsplit = (nt1 + g.tiles_per_split - 1) / g.tiles_per_split;
  g.rec = g.nsplit;  // the own keys ride in split 0
  return g;
}

size_t attention_ws_floats(bool bf16, int B, int H, int dh, int Tq, int L0, int L1, int kv1_bcast) {
  if (!bf16) return 0;
  if (use_groups(B, Tq, L0, L1, kv1_bcast)) {
    const GroupPlan g = group_plan(B, H, L0, L1);
    return g.rec > 1 ? (size_t)B * H * g.rec * Tq * (dh + 4) : 0;
  }
  AttnPlan p = attn_plan(B, H, Tq, L0, L1);
  return p.nsplit > 1 ? (size_t)B * H * p.nsplit * Tq * (dh + 4) : 0;
}

template <int DH, int QW, int KS, bool OWN = false>
static hipError_t run_attn(const AttnPlan& p, const bf16_t* q, const bf16_t* k0, const bf16_t* v0, int L0,
                           const bf16_t* k1, const bf16_t* v1, int L1, int B, int H, int Tq, bf16_t* o, float* ws,
                           hipStream_t s, int kv1_bcast, int groups = 0, int rec_nsplit = 0, int rec_base = 0,
                           const AttnPrefetch& pf = AttnPrefetch{}) {
  const int items = (groups > 0 ? H * groups : B * H * p.qtiles) * p.nsplit;
  if (rec_nsplit == 0) rec_nsplit = p.nsplit;
  const float scale_log2 = kLog2e / sqrtf((float)DH);
  // KS = 2: a 256-byte prefetch sink per wavefront after the stages
  const int lds = KS * 2 * (64 * DH * 2 + DH * 128) + (KS == 2 ? QW * KS * 256 : 0);
  auto kern = attn_bf16_mfma<DH, QW, KS, OWN>;
  static bool attr_set = false;  // per instantiation; the attribute is process-wide
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  kern<<<items, QW * KS * 64, lds, s>>>(q, k0, v0, L0, k1, v1, L1, B * H, H, Tq, p.qtiles, p.nsplit,
                                        p.tiles_per_split, scale_log2, o, rec_nsplit > 1 ? ws : nullptr, kv1_bcast,
                                        groups, rec_nsplit, rec_base, KS == 2 ? pf : AttnPrefetch{});
  return hipGetLastError();
}

// own keys (split 0), then the shared segment by sample groups
template <int DH>
static hipError_t run_grouped(const bf16_t* q, const bf16_t* k0, const bf16_t* v0, int L0, const bf16_t* k1,
                              const bf16_t* v1, int L1, int B, int H, int Tq, bf16_t* o, float* ws, hipStream_t s) {
  const GroupPlan g = group_plan(B, H, L0, L1);
  const AttnPlan shared{4, 2, 1, g.nsplit, g.tiles_per_split};
  return run_attn<DH, 4, 2, true>(shared, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s, 1, g.groups, g.rec, 0);
}

template <int DH>
static hipError_t run_attn_dh(const AttnPlan& p, const bf16_t* q, const bf16_t* k0, const bf16_t* v0, int L0,
                              const bf16_t* k1, const bf16_t* v1, int L1, int B, int H, int Tq, bf16_t* o,
                              float* ws, hipStream_t s, int kv1_bcast, const AttnPrefetch& pf) {
  if (p.qw == 1)
    return p.ks == 2 ? run_attn<DH, 1, 2>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s, kv1_bcast)
                     : run_attn<DH, 1, 1>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s, kv1_bcast);
  if (p.qw == 2) return run_attn<DH, 2, 1>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s, kv1_bcast);
  if (p.ks == 2) return run_attn<DH, 4, 2>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s, kv1_bcast, 0, 0, 0, pf);
  return run_attn<DH, 4, 1>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s, kv1_bcast);
}

static hipError_t launch_merge(const float* ws, int nsplit, int BH, int H, int Tq, int dh, bf16_t* o, hipStream_t s) {
  const int grid = (BH * Tq + 3) / 4;
  if (nsplit <= 4) attn_merge<bf16_t, 4><<<grid, 256, 0, s>>>(ws, nsplit, BH, H, Tq, dh, o);
  else if (nsplit <= 8) attn_merge<bf16_t, 8><<<grid, 256, 0, s>>>(ws, nsplit, BH, H, Tq, dh, o);
  else attn_merge<bf16_t, 16><<<grid, 256, 0, s>>>(ws, nsplit, BH, H, Tq, dh, o);
  return hipGetLastError();
}

template <class T>
hipError_t launch_attention(const T* q, const T* k0, const T* v0, int L0, const T* k1, const T* v1, int L1, int B,
                            int H, int dh, int Tq, T* o, float* ws, hipStream_t s, int kv1_bcast,
                            const AttnPrefetch& pf) {
  if (Tq <= 0 || B <= 0) return hipSuccess;
  if (L0 + L1 <= 0) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2) {
    if (use_groups(B, Tq, L0, L1, kv1_bcast)) {
      if (dh != 128 && dh != 64) return hipErrorInvalidValue;
      hipError_t e = dh == 128 ? run_grouped<128>(q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s)
                               : run_grouped<64>(q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s);
      const GroupPlan g = group_plan(B, H, L0, L1);
      if (e != hipSuccess || g.rec == 1) return e;
      return launch_merge(ws, g.rec, B * H, H, Tq, dh, o, s);
    }
    AttnPlan p = attn_plan(B, H, Tq, L0, L1);
    hipError_t e;
    if (dh == 128) e = run_attn_dh<128>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s, kv1_bcast, pf);
    else if (dh == 64) e = run_attn_dh<64>(p, q, k0, v0, L0, k1, v1, L1, B, H, Tq, o, ws, s, kv1_bcast, pf);
    else return hipErrorInvalidValue;
    if (e != hipSuccess || p.nsplit == 1) return e;
    return launch_merge(ws, p.nsplit, B * H, H, Tq, dh, o, s);
  } else {
    if (dh > 128) return hipErrorInvalidValue;
    dim3 grid((Tq + 3) / 4, B * H);
    attn_f32<<<grid, 256, 0, s>>>(q, k0, v0, L0, k1, v1, L1, H, Tq, dh, 1.0f / sqrtf((float)dh), o, kv1_bcast);
    return hipGetLastError();
  }
}

template hipError_t launch_attention<float>(const float*, const float*, const float*, int, const float*, const float*,
                                            int, int, int, int, int, float*, float*, hipStream_t, int,
                                            const AttnPrefetch&);
template hipError_t launch_attention<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*, int, const bf16_t*,
                                             const bf16_t*, int, int, int, int, int, bf16_t*, float*, hipStream_t, int,
                                             const AttnPrefetch&);
