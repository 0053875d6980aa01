// Fused continuous-filter convolution (CFConv), forward and backward.
//
// FlashSchNet §4.1 "Single-use edge pipeline" and §4.2 "Fused forward
// operator": per edge, the distance, the Gaussian basis with cosine envelope,
// the filter network and the gated message are produced and consumed on chip;
// §4.3 "Destination grouped segmented reduction": each destination owns a
// contiguous CSR segment and sums its messages without atomics; §4.3 "Source
// grouped segmented reduction in backward pass" gives the gradient of the
// source features, and §3.2 "Forces via autodiff" the force as the negative
// position gradient.
//
// Work decomposition (one work-group = 4 wave64, one per SIMD):
//  * a work-group owns a contiguous range of receivers, chosen so that all
//    groups get about the same number of edges + receivers (k_partition);
//  * it walks its edge range in tiles of 64 edges (two 32-row MFMA blocks;
//    tiles may straddle receivers);
//  * per tile: geometry in registers -> basis into LDS -> GEMM1 (basis x Wf1,
//    MFMA) -> shifted softplus into LDS -> GEMM2 (x Wf2, MFMA) -> gather of the
//    sender features in the MFMA output layout -> messages into LDS -> a
//    column-per-thread walk over the receivers of the tile that carries the
//    open receiver's partial sum into the next tile;
//  * the filter weights stay in LDS for the whole launch; no edge-sized
//    tensor ever reaches HBM.
//
// Backward (forces): the neighbour list is symmetric and w_ij = w_ji, so the
// owner of receiver i can produce, from its own row alone,
//   dE/dx_i   = dE/dx'_i + sum_j dE/dh_j * w_ij                (source sum)
//   dE/dd_ij  = filter-backward of (dE/dh_i * x_j + dE/dh_j * x_i)
//   dE/dr_i   = sum_j dE/dd_ij (r_i - r_j) / d_ij
// which needs no atomics: every output row has one owner. The forward filter
// is recomputed (nothing edge-sized was stored); dE/dd uses
// v = (d b~/dd) Wf1, computed with the same B operand as GEMM1, so
// dE/dd = sum_n (g_w Wf2^T)_n sigma(a)_n v_n.
//
// MFMA use: v_mfma_f32_32x32x2_f32 for fp32 filters, v_mfma_f32_32x32x16_bf16
// for bfloat16 filters. The k index inside each MFMA is permuted so every lane
// reads its A operand with one 16-byte LDS load (k = k0 + 4h + s for fp32,
// k = k0 + 8h + s for bf16, h = lane / 32); A and B use the same permutation.
#include "common.hpp"

namespace sn {

#define LN2F 0.69314718055994530942f

// ------------------------------------------------------------------ MFMA helpers
// acc[q] += A_q[32 x K] x B[K x 32] for NA independent A blocks sharing B.
// Ap[q] points at A_q row (lane % 32), column 4*(lane / 32); rows are 16-byte aligned.
// B[k][c] = W[k*SW + c0 + c] (BT = false) or W[(c0 + c)*SW + k] (BT = true).
template <int NA, bool BT>
__device__ __forceinline__ void mma_f32(f32x16* acc, const float* const* Ap, const float* W, int SW,
                                        int c0, int K, int lane) {
  const int h = lane >> 5, li = lane & 31;
  for (int k0 = 0; k0 < K; k0 += 8) {
    float b0, b1, b2, b3;
    if constexpr (BT) {
      const f32x4 bv = *reinterpret_cast<const f32x4*>(W + (c0 + li) * SW + k0 + 4 * h);
      b0 = bv.x; b1 = bv.y; b2 = bv.z; b3 = bv.w;
    } else {
      const float* wp = W + (k0 + 4 * h) * SW + c0 + li;
      b0 = wp[0]; b1 = wp[SW]; b2 = wp[2 * SW]; b3 = wp[3 * SW];
    }
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(Ap[q] + k0);
      acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, b0, acc[q], 0, 0, 0);
      acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, b1, acc[q], 0, 0, 0);
      acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, b2, acc[q], 0, 0, 0);
      acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, b3, acc[q], 0, 0, 0);
    }
  }
}

// bf16 operands: Ap[q] points at A_q row (lane % 32), column 8*(lane / 32);
// B[k][c] = Wt[(c0 + c)*SWt + k] (B stored transposed, k contiguous).
template <int NA>
__device__ __forceinline__ void mma_bf16(f32x16* acc, const __bf16* const* Ap, const __bf16* Wt,
                                         int SWt, int c0, int K, int lane) {
  const int h = lane >> 5, li = lane & 31;
  const __bf16* wp = Wt + (c0 + li) * SWt + 8 * h;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(wp + k0);
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ap[q] + k0);
      acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[q], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ int out_row(int r0, int r, int h) { return r0 + 8 * (r >> 2) + 4 * h + (r & 3); }

// Shifted softplus and its derivative from t = exp(-|a|).
__device__ __forceinline__ void ssp_sig(float a, float& s, float& sg) {
  const float t = __expf(-fabsf(a));
  const float inv = __builtin_amdgcn_rcpf(1.f + t);
  s = fmaxf(a, 0.f) + __logf(1.f + t) - LN2F;
  sg = a >= 0.f ? inv : t * inv;
}
__device__ __forceinline__ float ssp(float a) {
  const float t = __expf(-fabsf(a));
  return fmaxf(a, 0.f) + __logf(1.f + t) - LN2F;
}

__device__ __forceinline__ float min_image(float u, float box, float half) {
  if (u > half) return u - box;
  if (u < -half) return u + box;
  return u;
}

// ------------------------------------------------------------------ LDS plan
struct CfLds {
  int w1, w2, w2n;    // weight regions (bytes)
  int abuf;           // fp32 operand / staging region
  int hbuf;           // bf16 operand region
  int geo;            // per-edge geometry
  int total;
};

__host__ __device__ inline int align16(int b) { return (b + 15) & ~15; }

__host__ __device__ inline CfLds cf_plan(int D, int KP, bool bf16, bool bwd) {
  const int TM = kTileEdges;
  CfLds L{};
  int off = 0;
  if (bf16) {
    L.w1 = off; off += align16(D * (KP + 8) * 2);          // W1t [D][KP+8]
    L.w2 = off; off += align16(D * (D + 8) * 2);           // W2t [D][D+8]
    L.w2n = off; if (bwd) off += align16(D * (D + 8) * 2); // W2n [D][D+8]
    L.abuf = off; off += align16(TM * (D + 4) * 4);        // fp32 staging [TM][D+4]
    const int hb = (bwd ? 2 : 1) * TM * (KP + 8);
    L.hbuf = off; off += align16((hb > TM * (D + 8) ? hb : TM * (D + 8)) * 2);
  } else {
    L.w1 = off; off += align16(KP * (D + 4) * 4);          // W1s [KP][D+4]
    L.w2 = off; off += align16(D * (D + 4) * 4);           // W2s [D][D+4]
    L.w2n = L.w2;
    const int ab = (bwd ? 2 : 1) * TM * (KP + 4);
    L.abuf = off; off += align16((ab > TM * (D + 4) ? ab : TM * (D + 4)) * 4);
    L.hbuf = off;
  }
  L.geo = off; off += align16(TM * 13 * 4);
  L.total = off;
  return L;
}

int cf_kp(int Dr, int bf16) {
  const int m = bf16 ? 16 : 8;
  return (Dr + m - 1) / m * m;
}
size_t cf_lds_bytes(int D, int KP, int bf16, int backward) {
  return (size_t)cf_plan(D, KP, bf16 != 0, backward != 0).total;
}

// Per-edge geometry slots in LDS (TM each).
enum { G_D = 0, G_C, G_CP, G_IN, G_J, G_I, G_UX, G_UY, G_UZ, G_INVD, G_FX, G_FY, G_FZ, G_SLOTS };

template <int D, bool BF16, bool BWD>
__device__ __forceinline__ void stage_weights(const CfParams& p, unsigned char* lds, const CfLds& L) {
  const int KP = p.KP;
  if constexpr (BF16) {
    __bf16* W1t = reinterpret_cast<__bf16*>(lds + L.w1);
    __bf16* W2t = reinterpret_cast<__bf16*>(lds + L.w2);
    const __bf16* g1 = reinterpret_cast<const __bf16*>(p.W1t);
    const __bf16* g2 = reinterpret_cast<const __bf16*>(p.W2t);
    for (int idx = threadIdx.x; idx < D * KP; idx += kThreads) {
      const int n = idx / KP, k = idx - n * KP;
      W1t[n * (KP + 8) + k] = g1[idx];
    }
    for (int idx = threadIdx.x; idx < D * D; idx += kThreads) {
      const int n = idx / D, k = idx - n * D;
      W2t[n * (D + 8) + k] = g2[idx];
    }
    if constexpr (BWD) {
      __bf16* W2n = reinterpret_cast<__bf16*>(lds + L.w2n);
      const __bf16* g3 = reinterpret_cast<const __bf16*>(p.W2n);
      for (int idx = threadIdx.x; idx < D * D; idx += kThreads) {
        const int n = idx / D, k = idx - n * D;
        W2n[n * (D + 8) + k] = g3[idx];
      }
    }
  } else {
    float* W1s = reinterpret_cast<float*>(lds + L.w1);
    float* W2s = reinterpret_cast<float*>(lds + L.w2);
    for (int idx = threadIdx.x; idx < KP * D; idx += kThreads) {
      const int k = idx / D, n = idx - k * D;
      W1s[k * (D + 4) + n] = k < p.Dr ? p.Wf1[k * D + n] : 0.f;
    }
    for (int idx = threadIdx.x; idx < D * D; idx += kThreads) {
      const int k = idx / D, n = idx - k * D;
      W2s[k * (D + 4) + n] = p.Wf2[idx];
    }
  }
}

// Geometry of the tile's edges (threads 0..TM-1): receiver, sender, u = r_i - r_j,
// d, envelope and its derivative, and the inside-cutoff flag.
template <bool BWD>
__device__ __forceinline__ void tile_geometry(const CfParams& p, float* geo, int ts, int te, int cur) {
  const int TM = kTileEdges;
  const int r = threadIdx.x;
  if (r >= TM) return;
  const int e = ts + r;
  float d = 0.f, C = 0.f, Cp = 0.f, ux = 0.f, uy = 0.f, uz = 0.f, invd = 0.f;
  int j = 0, i = 0, inside = 0;
  if (e < te) {
    i = cur;
    while (p.rowptr[i + 1] <= e) ++i;
    j = p.col[e];
    ux = p.pos[3 * i + 0] - p.pos[3 * j + 0];
    uy = p.pos[3 * i + 1] - p.pos[3 * j + 1];
    uz = p.pos[3 * i + 2] - p.pos[3 * j + 2];
    if (p.periodic) {
      ux = min_image(ux, p.box, p.half_box);
      uy = min_image(uy, p.box, p.half_box);
      uz = min_image(uz, p.box, p.half_box);
    }
    d = sqrtf(ux * ux + uy * uy + uz * uz);
    inside = d < p.r_cut;
    if (inside) {
      float sn, cs;
      sincosf(p.pi_over_rc * d, &sn, &cs);
      C = 0.5f * (cs + 1.f);
      Cp = -0.5f * p.pi_over_rc * sn;
    }
    invd = d > 0.f ? 1.f / d : 0.f;
  }
  geo[G_D * TM + r] = d;
  geo[G_C * TM + r] = C;
  reinterpret_cast<int*>(geo)[G_IN * TM + r] = inside;
  reinterpret_cast<int*>(geo)[G_J * TM + r] = j;
  if constexpr (BWD) {
    geo[G_CP * TM + r] = Cp;
    reinterpret_cast<int*>(geo)[G_I * TM + r] = i;
    geo[G_UX * TM + r] = ux;
    geo[G_UY * TM + r] = uy;
    geo[G_UZ * TM + r] = uz;
    geo[G_INVD * TM + r] = invd;
  }
}

// Walk the receivers of one tile: add rows [lo, hi) of each receiver's part of
// the tile, and flush every receiver whose segment ends inside the tile.
template <class AddRows, class Flush>
__device__ __forceinline__ int seg_walk(const int32_t* rowptr, int cur, int ib, int ts, int te,
                                        AddRows add_rows, Flush flush) {
  int i = cur;
  while (i < ib) {
    const int rs = rowptr[i], re = rowptr[i + 1];
    const int lo = (rs > ts ? rs : ts) - ts, hi = (re < te ? re : te) - ts;
    add_rows(lo, hi);
    if (re > te) break;
    flush(i);
    ++i;
  }
  return i;
}

// ------------------------------------------------------------------ forward
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads, 1) void k_cf_fwd(CfParams p) {
  constexpr int TM = kTileEdges, NCB = D / 32, NRB = NCB / 2, SQ = D + 4, SW = D + 4, SH = D + 8;
  extern __shared__ __align__(16) unsigned char lds[];
  const int KP = p.KP;
  const CfLds L = cf_plan(D, KP, BF16, false);
  float* abuf = reinterpret_cast<float*>(lds + L.abuf);
  __bf16* hbuf = reinterpret_cast<__bf16*>(lds + L.hbuf);
  float* geo = reinterpret_cast<float*>(lds + L.geo);
  const int* geoi = reinterpret_cast<const int*>(geo);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, li = lane & 31;
  const int cb = wave % NCB, c = cb * 32 + li;
  int r0[NRB];
#pragma unroll
  for (int q = 0; q < NRB; ++q) r0[q] = (NRB == 2) ? 32 * q : 32 * (wave / NCB);

  stage_weights<D, BF16, false>(p, lds, L);
  const float bias1 = p.cf1[c], bias2 = p.cf2[c];
  const int ia = p.wg_start[blockIdx.x], ib = p.wg_start[blockIdx.x + 1];
  const int e_begin = p.rowptr[ia], e_end = p.rowptr[ib];
  int cur = ia;
  float acc_h = 0.f;
  __syncthreads();

  for (int ts = e_begin; ts < e_end; ts += TM) {
    const int te = min(ts + TM, e_end);
    tile_geometry<false>(p, geo, ts, te, cur);
    __syncthreads();
    // basis b~ = exp(-(d - mu_k)^2 / (2 sigma^2)) C(d), zero for padding and masked edges
    {
      const int SA = BF16 ? KP + 8 : KP + 4;
      for (int idx = tid; idx < TM * KP; idx += kThreads) {
        const int r = idx / KP, k = idx - r * KP;
        float v = 0.f;
        if (k < p.Dr && geoi[G_IN * TM + r]) {
          const float z = geo[G_D * TM + r] - (p.rbf_min + (float)k * p.rbf_step);
          v = __expf(p.rbf_coef * z * z) * geo[G_C * TM + r];
        }
        if constexpr (BF16) hbuf[r * SA + k] = (__bf16)v;
        else abuf[r * SA + k] = v;
      }
    }
    __syncthreads();
    f32x16 acc[NRB];
#pragma unroll
    for (int q = 0; q < NRB; ++q) acc[q] = f32x16{};
    if constexpr (BF16) {
      const __bf16* Ap[NRB];
      for (int q = 0; q < NRB; ++q) Ap[q] = hbuf + (r0[q] + li) * (KP + 8) + 8 * h;
      mma_bf16<NRB>(acc, Ap, reinterpret_cast<const __bf16*>(lds + L.w1), KP + 8, cb * 32, KP, lane);
    } else {
      const float* Ap[NRB];
      for (int q = 0; q < NRB; ++q) Ap[q] = abuf + (r0[q] + li) * (KP + 4) + 4 * h;
      mma_f32<NRB, false>(acc, Ap, reinterpret_cast<const float*>(lds + L.w1), SW, cb * 32, KP, lane);
    }
    __syncthreads();
    // s = ssp(a), the A operand of the second filter layer
#pragma unroll
    for (int q = 0; q < NRB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = out_row(r0[q], r, h);
        const float s = ssp(acc[q][r] + bias1);
        if constexpr (BF16) hbuf[row * SH + c] = (__bf16)s;
        else abuf[row * SQ + c] = s;
        acc[q][r] = 0.f;
      }
    __syncthreads();
    if constexpr (BF16) {
      const __bf16* Ap[NRB];
      for (int q = 0; q < NRB; ++q) Ap[q] = hbuf + (r0[q] + li) * SH + 8 * h;
      mma_bf16<NRB>(acc, Ap, reinterpret_cast<const __bf16*>(lds + L.w2), SH, cb * 32, D, lane);
    } else {
      const float* Ap[NRB];
      for (int q = 0; q < NRB; ++q) Ap[q] = abuf + (r0[q] + li) * SQ + 4 * h;
      mma_f32<NRB, false>(acc, Ap, reinterpret_cast<const float*>(lds + L.w2), SW, cb * 32, D, lane);
    }
    __syncthreads();
    // m = x_src * w, gathered in the MFMA output layout
#pragma unroll
    for (int q = 0; q < NRB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = out_row(r0[q], r, h);
        const float w = geoi[G_IN * TM + row] ? acc[q][r] + bias2 : 0.f;
        abuf[row * SQ + c] = w * p.x[(size_t)geoi[G_J * TM + row] * D + c];
      }
    __syncthreads();
    cur = seg_walk(
        p.rowptr, cur, ib, ts, te,
        [&](int lo, int hi) {
          if (tid < D)
            for (int r = lo; r < hi; ++r) acc_h += abuf[r * SQ + tid];
        },
        [&](int i) {
          if (tid < D) p.h[(size_t)i * D + tid] = acc_h;
          acc_h = 0.f;
        });
    __syncthreads();
  }
  for (; cur < ib; ++cur)
    if (tid < D) p.h[(size_t)cur * D + tid] = 0.f;
}

// ------------------------------------------------------------------ backward
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads, 1) void k_cf_bwd(CfParams p) {
  constexpr int TM = kTileEdges, NCB = D / 32, NRB = NCB / 2, SQ = D + 4, SW = D + 4, SH = D + 8;
  extern __shared__ __align__(16) unsigned char lds[];
  const int KP = p.KP;
  const CfLds L = cf_plan(D, KP, BF16, true);
  float* abuf = reinterpret_cast<float*>(lds + L.abuf);
  __bf16* hbuf = reinterpret_cast<__bf16*>(lds + L.hbuf);
  float* geo = reinterpret_cast<float*>(lds + L.geo);
  const int* geoi = reinterpret_cast<const int*>(geo);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, li = lane & 31;
  const int cb = wave % NCB, c = cb * 32 + li;
  int r0[NRB];
#pragma unroll
  for (int q = 0; q < NRB; ++q) r0[q] = (NRB == 2) ? 32 * q : 32 * (wave / NCB);

  stage_weights<D, BF16, true>(p, lds, L);
  const float bias1 = p.cf1[c], bias2 = p.cf2[c];
  const int ia = p.wg_start[blockIdx.x], ib = p.wg_start[blockIdx.x + 1];
  const int e_begin = p.rowptr[ia], e_end = p.rowptr[ib];
  const bool want_gx = p.gx_out != nullptr;
  int cur = ia;
  float acc_q = 0.f, acc_f = 0.f;
  __syncthreads();

  for (int ts = e_begin; ts < e_end; ts += TM) {
    const int te = min(ts + TM, e_end);
    tile_geometry<true>(p, geo, ts, te, cur);
    __syncthreads();
    // b~ and d b~ / dd
    {
      const int SA = BF16 ? KP + 8 : KP + 4;
      for (int idx = tid; idx < TM * KP; idx += kThreads) {
        const int r = idx / KP, k = idx - r * KP;
        float bt = 0.f, btp = 0.f;
        if (k < p.Dr && geoi[G_IN * TM + r]) {
          const float z = geo[G_D * TM + r] - (p.rbf_min + (float)k * p.rbf_step);
          const float g = __expf(p.rbf_coef * z * z);
          const float C = geo[G_C * TM + r], Cp = geo[G_CP * TM + r];
          bt = g * C;
          btp = g * (Cp - z * p.rbf_inv_s2 * C);
        }
        if constexpr (BF16) {
          hbuf[r * SA + k] = (__bf16)bt;
          hbuf[(TM + r) * SA + k] = (__bf16)btp;
        } else {
          abuf[r * SA + k] = bt;
          abuf[(TM + r) * SA + k] = btp;
        }
      }
    }
    __syncthreads();
    // GEMM1 on both operands: a = b~ Wf1, v = (d b~/dd) Wf1
    f32x16 acc[2 * NRB];
#pragma unroll
    for (int q = 0; q < 2 * NRB; ++q) acc[q] = f32x16{};
    if constexpr (BF16) {
      const __bf16* Ap[2 * NRB];
      for (int q = 0; q < NRB; ++q) {
        Ap[q] = hbuf + (r0[q] + li) * (KP + 8) + 8 * h;
        Ap[NRB + q] = hbuf + (TM + r0[q] + li) * (KP + 8) + 8 * h;
      }
      mma_bf16<2 * NRB>(acc, Ap, reinterpret_cast<const __bf16*>(lds + L.w1), KP + 8, cb * 32, KP,
                        lane);
    } else {
      const float* Ap[2 * NRB];
      for (int q = 0; q < NRB; ++q) {
        Ap[q] = abuf + (r0[q] + li) * (KP + 4) + 4 * h;
        Ap[NRB + q] = abuf + (TM + r0[q] + li) * (KP + 4) + 4 * h;
      }
      mma_f32<2 * NRB, false>(acc, Ap, reinterpret_cast<const float*>(lds + L.w1), SW, cb * 32, KP,
                              lane);
    }
    __syncthreads();
    // s = ssp(a) -> LDS; keep sigma(a) in acc[q] and v in acc[NRB + q]
#pragma unroll
    for (int q = 0; q < NRB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = out_row(r0[q], r, h);
        float s, sg;
        ssp_sig(acc[q][r] + bias1, s, sg);
        acc[q][r] = sg;
        if constexpr (BF16) hbuf[row * SH + c] = (__bf16)s;
        else abuf[row * SQ + c] = s;
      }
    __syncthreads();
    f32x16 accw[NRB];
#pragma unroll
    for (int q = 0; q < NRB; ++q) accw[q] = f32x16{};
    if constexpr (BF16) {
      const __bf16* Ap[NRB];
      for (int q = 0; q < NRB; ++q) Ap[q] = hbuf + (r0[q] + li) * SH + 8 * h;
      mma_bf16<NRB>(accw, Ap, reinterpret_cast<const __bf16*>(lds + L.w2), SH, cb * 32, D, lane);
    } else {
      const float* Ap[NRB];
      for (int q = 0; q < NRB; ++q) Ap[q] = abuf + (r0[q] + li) * SQ + 4 * h;
      mma_f32<NRB, false>(accw, Ap, reinterpret_cast<const float*>(lds + L.w2), SW, cb * 32, D,
                          lane);
    }
    __syncthreads();
    // gathers; q = dE/dh_j * w (source sum), g_w = dE/dh_i * x_j + dE/dh_j * x_i (both directions)
    f32x16 gw[NRB];
#pragma unroll
    for (int q = 0; q < NRB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = out_row(r0[q], r, h);
        const bool in = geoi[G_IN * TM + row] != 0;
        const size_t j = (size_t)geoi[G_J * TM + row], i = (size_t)geoi[G_I * TM + row];
        const float w = in ? accw[q][r] + bias2 : 0.f;
        const float xj = p.x[j * D + c], ghj = p.gh[j * D + c];
        const float xi = p.x[i * D + c], ghi = p.gh[i * D + c];
        accw[q][r] = ghj * w;
        gw[q][r] = in ? ghi * xj + ghj * xi : 0.f;
      }
    if (want_gx) {
#pragma unroll
      for (int q = 0; q < NRB; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) abuf[out_row(r0[q], r, h) * SQ + c] = accw[q][r];
      __syncthreads();
      seg_walk(
          p.rowptr, cur, ib, ts, te,
          [&](int lo, int hi) {
            if (tid < D)
              for (int r = lo; r < hi; ++r) acc_q += abuf[r * SQ + tid];
          },
          [&](int i) {
            if (tid < D) p.gx_out[(size_t)i * D + tid] = p.gx_in[(size_t)i * D + tid] + acc_q;
            acc_q = 0.f;
          });
      __syncthreads();
    }
    // g_w -> LDS, GEMM3: g_s = g_w Wf2^T
#pragma unroll
    for (int q = 0; q < NRB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = out_row(r0[q], r, h);
        if constexpr (BF16) hbuf[row * SH + c] = (__bf16)gw[q][r];
        else abuf[row * SQ + c] = gw[q][r];
        gw[q][r] = 0.f;
      }
    __syncthreads();
    if constexpr (BF16) {
      const __bf16* Ap[NRB];
      for (int q = 0; q < NRB; ++q) Ap[q] = hbuf + (r0[q] + li) * SH + 8 * h;
      mma_bf16<NRB>(gw, Ap, reinterpret_cast<const __bf16*>(lds + L.w2n), SH, cb * 32, D, lane);
    } else {
      const float* Ap[NRB];
      for (int q = 0; q < NRB; ++q) Ap[q] = abuf + (r0[q] + li) * SQ + 4 * h;
      mma_f32<NRB, true>(gw, Ap, reinterpret_cast<const float*>(lds + L.w2), SW, cb * 32, D, lane);
    }
    __syncthreads();
    // p = g_s * sigma(a) * v, summed over features per edge -> dE/dd
#pragma unroll
    for (int q = 0; q < NRB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        abuf[out_row(r0[q], r, h) * SQ + c] = gw[q][r] * acc[q][r] * acc[NRB + q][r];
    __syncthreads();
    {
      const int r = tid >> 2, part = tid & 3;
      float s = 0.f;
      const float* rowp = abuf + r * SQ + part * (D / 4);
#pragma unroll 8
      for (int k = 0; k < D / 4; ++k) s += rowp[k];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      if (part == 0) {
        const float gd = geoi[G_IN * TM + r] ? s * geo[G_INVD * TM + r] : 0.f;
        geo[G_FX * TM + r] = gd * geo[G_UX * TM + r];
        geo[G_FY * TM + r] = gd * geo[G_UY * TM + r];
        geo[G_FZ * TM + r] = gd * geo[G_UZ * TM + r];
      }
    }
    __syncthreads();
    cur = seg_walk(
        p.rowptr, cur, ib, ts, te,
        [&](int lo, int hi) {
          if (tid < 3)
            for (int r = lo; r < hi; ++r)
              acc_f += geo[(G_FX + tid) * TM + r];
        },
        [&](int i) {
          if (tid < 3) {
            float* f = p.forces + (size_t)i * 3 + tid;
            *f = (p.force_accumulate ? *f : 0.f) - acc_f;
          }
          acc_f = 0.f;
        });
    __syncthreads();
  }
  for (; cur < ib; ++cur) {
    if (want_gx && tid < D) p.gx_out[(size_t)cur * D + tid] = p.gx_in[(size_t)cur * D + tid];
    if (tid < 3 && !p.force_accumulate) p.forces[(size_t)cur * 3 + tid] = 0.f;
  }
}

// ------------------------------------------------------------------ partition
// Work-group w owns receivers [wg_start[w], wg_start[w+1]); boundaries split
// the monotone key rowptr[i] + i (edges plus one unit per receiver) evenly.
__global__ void k_partition(const int32_t* rowptr, int N, int G, int32_t* wg_start) {
  const int w = blockIdx.x * blockDim.x + threadIdx.x;
  if (w > G) return;
  if (w == 0) { wg_start[0] = 0; return; }
  if (w == G) { wg_start[G] = N; return; }
  const int64_t total = (int64_t)rowptr[N] + N;
  const int64_t target = (total * w + G - 1) / G;
  int lo = 0, hi = N;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)rowptr[mid] + mid >= target) hi = mid;
    else lo = mid + 1;
  }
  wg_start[w] = lo;
}

hipError_t launch_partition(const int32_t* rowptr, int n_atoms, int G, int32_t* wg_start,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_partition, dim3((G + 1 + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                     rowptr, n_atoms, G, wg_start);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t set_lds_limit() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_cf_fwd<D, BF16>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_cf_bwd<D, BF16>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

hipError_t cf_prepare(int D, int bf16) {
  if (D == 64) return bf16 ? set_lds_limit<64, true>() : set_lds_limit<64, false>();
  if (D == 128) return bf16 ? set_lds_limit<128, true>() : set_lds_limit<128, false>();
  return hipErrorInvalidValue;
}

#define SN_CF_DISPATCH(KERNEL, BWD)                                                              \
  do {                                                                                           \
    const size_t lds = cf_lds_bytes(D, p.KP, bf16, BWD);                                         \
    if (D == 64 && !bf16) hipLaunchKernelGGL((KERNEL<64, false>), dim3(G), dim3(kThreads), lds, s, p); \
    else if (D == 64) hipLaunchKernelGGL((KERNEL<64, true>), dim3(G), dim3(kThreads), lds, s, p); \
    else if (!bf16) hipLaunchKernelGGL((KERNEL<128, false>), dim3(G), dim3(kThreads), lds, s, p); \
    else hipLaunchKernelGGL((KERNEL<128, true>), dim3(G), dim3(kThreads), lds, s, p);            \
  } while (0)

hipError_t launch_cf_forward(int D, int bf16, const CfParams& p, int G, hipStream_t s) {
  SN_CF_DISPATCH(k_cf_fwd, 0);
  return hipGetLastError();
}

hipError_t launch_cf_backward(int D, int bf16, const CfParams& p, int G, hipStream_t s) {
  SN_CF_DISPATCH(k_cf_bwd, 1);
  return hipGetLastError();
}

} // namespace sn
