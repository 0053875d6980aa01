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
// Work decomposition (one work-group = 8 wave64, two per SIMD, so one wave's
// elementwise work overlaps the other's matrix work):
//  * a work-group owns a contiguous range of receivers, chosen so that all
//    groups get about the same number of edges + receivers (k_partition); its
//    slice of rowptr is staged in LDS;
//  * it walks its edge range in tiles of TM edges (TM = 64 for D = 128,
//    128 for D = 64, so a tile is always eight 32x32 output blocks, one per
//    wave); tiles may straddle receivers;
//  * per tile: geometry -> basis into LDS -> GEMM1 (basis x Wf1, MFMA) ->
//    shifted softplus into LDS -> GEMM2 (x Wf2, MFMA) -> gather of the sender
//    features in the MFMA output layout -> messages into LDS -> segmented sum:
//    every receiver of the tile is summed by its own thread group in
//    parallel; the receiver open at the tile's end leaves its partial sum in a
//    double-buffered carry row for the next tile;
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
// dE/dd = sum_n (g_w Wf2^T)_n sigmoid(a)_n v_n.
//
// MFMA use: v_mfma_f32_32x32x2_f32 for fp32 filters, v_mfma_f32_32x32x16_bf16
// for bfloat16 filters. The k index inside each MFMA is permuted so every lane
// reads its A operand with one 16-byte LDS load (k = k0 + 4h + s for fp32,
// k = k0 + 8h + s for bf16, h = lane / 32); A and B use the same permutation.
// Gathers use buffer loads with 32-bit byte offsets.
#include <type_traits>

#include "common.hpp"

namespace sn {

#define LN2F 0.69314718055994530942f
#define LOG2EF 1.44269504088896340736f

constexpr int kCfThreads = 512;
constexpr int kRpMax = 2048;    // rowptr entries of a work-group staged in LDS

template <int D> struct CfShape { static constexpr int TM = D == 128 ? 64 : 128; };

// ------------------------------------------------------------------ small helpers
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float bload(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ int bload_i(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}

// e^x for x <= 0 and ln(y) for y in [1, 2], on the hardware exp2 / log2.
__device__ __forceinline__ float exp_neg(float x) { return __builtin_amdgcn_exp2f(x * LOG2EF); }
__device__ __forceinline__ float ln_1_2(float y) { return __builtin_amdgcn_logf(y) * LN2F; }

// Shifted softplus and its derivative from t = exp(-|a|).
__device__ __forceinline__ void ssp_sig(float a, float& s, float& sg) {
  const float t = exp_neg(-fabsf(a));
  const float inv = __builtin_amdgcn_rcpf(1.f + t);
  s = fmaxf(a, 0.f) + ln_1_2(1.f + t) - LN2F;
  sg = a >= 0.f ? inv : t * inv;
}
__device__ __forceinline__ float ssp(float a) {
  const float t = exp_neg(-fabsf(a));
  return fmaxf(a, 0.f) + ln_1_2(1.f + t) - LN2F;
}

__device__ __forceinline__ float min_image(float u, float box, float half) {
  if (u > half) return u - box;
  if (u < -half) return u + box;
  return u;
}

__device__ __forceinline__ int out_row(int r0, int r, int h) { return r0 + 8 * (r >> 2) + 4 * h + (r & 3); }

// ------------------------------------------------------------------ MFMA helpers
// acc[q] += A_q[32 x K] x B[K x 32] for NA A blocks sharing B.
// Ap[q] points at A_q row (lane % 32), column 4*(lane / 32); rows 16-byte aligned.
// B[k][c] = W[k*SW + c0 + c] (BT = false) or W[(c0 + c)*SW + k] (BT = true).
template <int NA, bool BT, int K>
__device__ __forceinline__ void mma_f32(f32x16* acc, const float* const* Ap, const float* W, int SW,
                                        int c0, int lane) {
  const int h = lane >> 5, li = lane & 31;
#pragma unroll 2
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
template <int NA, int K>
__device__ __forceinline__ void mma_bf16(f32x16* acc, const __bf16* const* Ap, const __bf16* Wt,
                                         int SWt, int c0, int lane) {
  const int h = lane >> 5, li = lane & 31;
  const __bf16* wp = Wt + (c0 + li) * SWt + 8 * h;
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += 16) {
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(wp + k0);
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ap[q] + k0);
      acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[q], 0, 0, 0);
    }
  }
}

// ------------------------------------------------------------------ LDS plan
struct CfLds {
  int w1, w2, w2n;    // weight regions (bytes)
  int abuf;           // fp32 operand / staging region
  int hbuf;           // bf16 operand region
  int geo;            // per-edge geometry
  int rp;             // rowptr slice
  int carry;          // carry rows of the segmented sums
  int total;
};

enum { G_D = 0, G_C, G_CP, G_IN, G_J, G_I, G_UX, G_UY, G_UZ, G_INVD, G_FX, G_FY, G_FZ, G_SLOTS };

__host__ __device__ inline int align16(int b) { return (b + 15) & ~15; }

__host__ __device__ inline CfLds cf_plan(int D, int KP, bool bf16, bool bwd) {
  const int TM = D == 128 ? 64 : 128;
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
  L.geo = off; off += align16(TM * G_SLOTS * 4);
  L.rp = off; off += align16(kRpMax * 4);
  L.carry = off; off += align16((bwd ? 2 * D + 8 : 2 * D) * 4);
  L.total = off;
  return L;
}

int cf_kp(int Dr, int bf16) {
  if (Dr <= 32) return 32;
  if (!bf16 && Dr <= 56) return 56;
  return 64;
}
size_t cf_lds_bytes(int D, int KP, int bf16, int backward) {
  return (size_t)cf_plan(D, KP, bf16 != 0, backward != 0).total;
}

// ------------------------------------------------------------------ shared pieces
template <int D, int KP, bool BF16, bool BWD>
__device__ __forceinline__ void stage_weights(const CfParams& p, unsigned char* lds, const CfLds& L) {
  if constexpr (BF16) {
    // global copies are compact [D][KP] and [D][D]; 8 bf16 (16 bytes) per move
    const f32x4* g1 = reinterpret_cast<const f32x4*>(p.W1t);
    const f32x4* g2 = reinterpret_cast<const f32x4*>(p.W2t);
    for (int idx = threadIdx.x; idx < D * KP / 8; idx += kCfThreads) {
      const int n = idx / (KP / 8), k8 = idx - n * (KP / 8);
      *reinterpret_cast<f32x4*>(lds + L.w1 + (n * (KP + 8) + 8 * k8) * 2) = g1[idx];
    }
    for (int idx = threadIdx.x; idx < D * D / 8; idx += kCfThreads) {
      const int n = idx / (D / 8), k8 = idx - n * (D / 8);
      *reinterpret_cast<f32x4*>(lds + L.w2 + (n * (D + 8) + 8 * k8) * 2) = g2[idx];
    }
    if constexpr (BWD) {
      const f32x4* g3 = reinterpret_cast<const f32x4*>(p.W2n);
      for (int idx = threadIdx.x; idx < D * D / 8; idx += kCfThreads) {
        const int n = idx / (D / 8), k8 = idx - n * (D / 8);
        *reinterpret_cast<f32x4*>(lds + L.w2n + (n * (D + 8) + 8 * k8) * 2) = g3[idx];
      }
    }
  } else {
    float* W1s = reinterpret_cast<float*>(lds + L.w1);
    float* W2s = reinterpret_cast<float*>(lds + L.w2);
    const f32x4* g1 = reinterpret_cast<const f32x4*>(p.Wf1);
    const f32x4* g2 = reinterpret_cast<const f32x4*>(p.Wf2);
    for (int idx = threadIdx.x; idx < KP * D / 4; idx += kCfThreads) {
      const int k = idx / (D / 4), n4 = idx - k * (D / 4);
      const f32x4 v = k < p.Dr ? g1[idx] : f32x4{};
      *reinterpret_cast<f32x4*>(W1s + k * (D + 4) + 4 * n4) = v;
    }
    for (int idx = threadIdx.x; idx < D * D / 4; idx += kCfThreads) {
      const int k = idx / (D / 4), n4 = idx - k * (D / 4);
      *reinterpret_cast<f32x4*>(W2s + k * (D + 4) + 4 * n4) = g2[idx];
    }
  }
}

// rowptr access: FULL when the work-group's whole slice sits in LDS (the
// common case; no global loads, so the compiler need not drain in-flight
// prefetches), else through the slice when the index falls inside it.
template <bool FULL>
struct RowPtr {
  const int32_t* g;
  const int32_t* s;
  int base, len;
  __device__ __forceinline__ int operator()(int i) const {
    const int k = i - base;
    if constexpr (FULL) return s[k];
    return k < len ? s[k] : g[i];
  }
};

// Geometry loads run one tile ahead of the arithmetic: while tile k computes,
// the positions of tile k+1 and the sender indices of tile k+2 are in flight
// (threads 0..TM-1, one edge each).
struct GeoPrefetch {
  int i, j, jn;                 // receiver and sender of the next tile's edge; sender a tile later
  float xi, yi, zi, xj, yj, zj; // their positions
};

__device__ __forceinline__ void pf_positions(GeoPrefetch& f, __amdgpu_buffer_rsrc_t rpos) {
  const uint32_t oi = (uint32_t)f.i * 12u, oj = (uint32_t)f.j * 12u;
  f.xi = bload(rpos, oi);
  f.yi = bload(rpos, oi + 4);
  f.zi = bload(rpos, oi + 8);
  f.xj = bload(rpos, oj);
  f.yj = bload(rpos, oj + 4);
  f.zj = bload(rpos, oj + 8);
}

template <int TM, class RPT>
__device__ __forceinline__ void pf_start(GeoPrefetch& f, const RPT& RP, int ia, int ts, int e_end,
                                         __amdgpu_buffer_rsrc_t rcol, __amdgpu_buffer_rsrc_t rpos) {
  const int e = ts + (int)threadIdx.x, e2 = e + TM;
  // reads past the last edge return 0 (the buffer descriptor bounds them)
  f.j = bload_i(rcol, (uint32_t)e * 4u);
  f.jn = bload_i(rcol, (uint32_t)e2 * 4u);
  int i = ia;
  if (e < e_end)
    while (RP(i + 1) <= e) ++i;
  f.i = i;
  pf_positions(f, rpos);
}

// Move the prefetch on to the tile starting at ts (the previous tile's values
// have been consumed).
template <int TM, class RPT>
__device__ __forceinline__ void pf_advance(GeoPrefetch& f, const RPT& RP, int ts, int e_end,
                                           __amdgpu_buffer_rsrc_t rcol,
                                           __amdgpu_buffer_rsrc_t rpos) {
  const int e = ts + (int)threadIdx.x, e2 = e + TM;
  int i = f.i;
  if (e < e_end)
    while (RP(i + 1) <= e) ++i;
  f.i = i;
  f.j = f.jn;
  f.jn = bload_i(rcol, (uint32_t)e2 * 4u);
  pf_positions(f, rpos);
}

// Geometry of the tile's edges from the prefetched values (threads 0..TM-1):
// receiver, sender, u = r_i - r_j, d, envelope and its derivative, and the
// inside-cutoff flag. Rows past the tile end get receiver `cur`, sender 0.
template <int TM, bool BWD>
__device__ __forceinline__ void tile_geometry(const CfParams& p, const GeoPrefetch& f, float* geo,
                                              int ts, int te, int cur) {
  const int r = threadIdx.x;
  const int e = ts + r;
  float d = 0.f, C = 0.f, Cp = 0.f, ux = 0.f, uy = 0.f, uz = 0.f, invd = 0.f;
  int j = 0, i = cur, inside = 0;
  if (e < te) {
    i = f.i;
    j = f.j;
    ux = f.xi - f.xj;
    uy = f.yi - f.yj;
    uz = f.zi - f.zj;
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
  int* geoi = reinterpret_cast<int*>(geo);
  geo[G_D * TM + r] = d;
  geo[G_C * TM + r] = C;
  geoi[G_IN * TM + r] = inside;
  geoi[G_J * TM + r] = j;
  geoi[G_I * TM + r] = i;
  if constexpr (BWD) {
    geo[G_CP * TM + r] = Cp;
    geo[G_UX * TM + r] = ux;
    geo[G_UY * TM + r] = uy;
    geo[G_UZ * TM + r] = uz;
    geo[G_INVD * TM + r] = invd;
  }
}

// The receivers [first, last] of a tile; `last_open` when the last one's
// segment continues into the next tile.
struct TileSegs {
  int first, last, nseg;
  bool last_open;
};
template <int TM, class RPT>
__device__ __forceinline__ TileSegs tile_segs(const RPT& RP, const int* geoi, int ts, int te,
                                              int cur) {
  TileSegs t;
  t.first = cur;
  t.last = geoi[G_I * TM + (te - ts - 1)];
  t.nseg = t.last - t.first + 1;
  t.last_open = RP(t.last + 1) > te;
  return t;
}

// Column-parallel segmented sum of the tile rows in `buf` (stride SQ): every
// receiver of the tile gets one thread per column; the first receiver adds the
// carried partial sum, the last one either stores its partial (still open) or
// clears the carry. flush(i, c, value) writes a completed receiver.
template <int D, int SQ, class RPT, class Flush>
__device__ __forceinline__ void seg_sum_cols(const RPT& RP, const TileSegs& t, int ts, int te,
                                             const float* buf, const float* carry_in,
                                             float* carry_out, Flush flush) {
  constexpr int NG = kCfThreads / D;
  const int g = threadIdx.x / D, c = threadIdx.x - g * D;
  for (int k = g; k < t.nseg; k += NG) {
    const int i = t.first + k;
    const int rs = RP(i), re = RP(i + 1);
    const int lo = (rs > ts ? rs : ts) - ts, hi = (re < te ? re : te) - ts;
    float s = 0.f;
    for (int r = lo; r < hi; ++r) s += buf[r * SQ + c];
    if (k == 0) s += carry_in[c];
    if (k == t.nseg - 1) {
      if (t.last_open) {
        carry_out[c] = s;
        continue;
      }
      carry_out[c] = 0.f;
    }
    flush(i, c, s);
  }
}

// ------------------------------------------------------------------ forward
template <int D, int KP, bool BF16>
__global__ __launch_bounds__(kCfThreads, 1) void k_cf_fwd(CfParams p) {
  constexpr int TM = CfShape<D>::TM, NCB = D / 32, SQ = D + 4, SW = D + 4, SH = D + 8;
  constexpr int SA = BF16 ? KP + 8 : KP + 4;
  extern __shared__ __align__(16) unsigned char lds[];
  const CfLds L = cf_plan(D, KP, BF16, false);
  float* abuf = reinterpret_cast<float*>(lds + L.abuf);
  __bf16* hbuf = reinterpret_cast<__bf16*>(lds + L.hbuf);
  float* geo = reinterpret_cast<float*>(lds + L.geo);
  const int* geoi = reinterpret_cast<const int*>(geo);
  int32_t* rps = reinterpret_cast<int32_t*>(lds + L.rp);
  float* carry = reinterpret_cast<float*>(lds + L.carry);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, li = lane & 31;
  const int cb = wave % NCB, r0 = 32 * (wave / NCB), c = cb * 32 + li;
  const uint32_t N = (uint32_t)p.n_atoms;
  const __amdgpu_buffer_rsrc_t rcol = rsrc(p.col, (uint32_t)p.rowptr[p.n_atoms] * 4u);
  const __amdgpu_buffer_rsrc_t rpos = rsrc(p.pos, N * 12u);
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, N * (uint32_t)D * 4u);

  stage_weights<D, KP, BF16, false>(p, lds, L);
  const float bias1 = p.cf1[c], bias2 = p.cf2[c];
  const int ia = p.wg_start[blockIdx.x], ib = p.wg_start[blockIdx.x + 1];
  const int rpl = min(ib - ia + 1, kRpMax);
  for (int k = tid; k < rpl; k += kCfThreads) rps[k] = p.rowptr[ia + k];
  for (int k = tid; k < 2 * D; k += kCfThreads) carry[k] = 0.f;
  __syncthreads();
  auto tiles = [&](auto full) {
  const RowPtr<decltype(full)::value> RP{p.rowptr, rps, ia, rpl};
  const int e_begin = RP(ia), e_end = RP(ib);
  int cur = ia, par = 0;
  GeoPrefetch pf{};
  if (tid < TM) pf_start<TM>(pf, RP, ia, e_begin, e_end, rcol, rpos);

  for (int ts = e_begin; ts < e_end; ts += TM) {
    const int te = min(ts + TM, e_end);
    if (tid < TM) {
      tile_geometry<TM, false>(p, pf, geo, ts, te, cur);
      pf_advance<TM>(pf, RP, ts + TM, e_end, rcol, rpos);
    }
    __syncthreads();
    // sender features, needed after the filter: issue the gathers now
    float xg[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      xg[r] = bload(rx, ((uint32_t)geoi[G_J * TM + out_row(r0, r, h)] * D + c) * 4u);
    // basis b~ = exp(-(d - mu_k)^2 / (2 sigma^2)) C(d), zero for padding and masked edges
    for (int idx = tid; idx < TM * KP; idx += kCfThreads) {
      const int r = idx / KP, k = idx - r * KP;
      float v = 0.f;
      if (k < p.Dr && geoi[G_IN * TM + r]) {
        const float z = geo[G_D * TM + r] - (p.rbf_min + (float)k * p.rbf_step);
        v = __builtin_amdgcn_exp2f(p.rbf_coef2 * z * z) * geo[G_C * TM + r];
      }
      if constexpr (BF16) hbuf[r * SA + k] = (__bf16)v;
      else abuf[r * SA + k] = v;
    }
    __syncthreads();
    f32x16 acc[1] = {f32x16{}};
    if constexpr (BF16) {
      const __bf16* Ap[1] = {hbuf + (r0 + li) * SA + 8 * h};
      mma_bf16<1, KP>(acc, Ap, reinterpret_cast<const __bf16*>(lds + L.w1), SA, cb * 32, lane);
    } else {
      const float* Ap[1] = {abuf + (r0 + li) * SA + 4 * h};
      mma_f32<1, false, KP>(acc, Ap, reinterpret_cast<const float*>(lds + L.w1), SW, cb * 32, lane);
    }
    __syncthreads();
    // s = ssp(a), the A operand of the second filter layer
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = out_row(r0, r, h);
      const float s = ssp(acc[0][r] + bias1);
      if constexpr (BF16) hbuf[row * SH + c] = (__bf16)s;
      else abuf[row * SQ + c] = s;
      acc[0][r] = 0.f;
    }
    __syncthreads();
    if constexpr (BF16) {
      const __bf16* Ap[1] = {hbuf + (r0 + li) * SH + 8 * h};
      mma_bf16<1, D>(acc, Ap, reinterpret_cast<const __bf16*>(lds + L.w2), SH, cb * 32, lane);
    } else {
      const float* Ap[1] = {abuf + (r0 + li) * SQ + 4 * h};
      mma_f32<1, false, D>(acc, Ap, reinterpret_cast<const float*>(lds + L.w2), SW, cb * 32, lane);
    }
    // m = x_src * w in the MFMA output layout
    float m[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = out_row(r0, r, h);
      const float mk = geoi[G_IN * TM + row] ? 1.f : 0.f;
      m[r] = mk * ((acc[0][r] + bias2) * xg[r]);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) abuf[out_row(r0, r, h) * SQ + c] = m[r];
    __syncthreads();
    const TileSegs t = tile_segs<TM>(RP, geoi, ts, te, cur);
    seg_sum_cols<D, SQ>(RP, t, ts, te, abuf, carry + par * D, carry + (1 - par) * D,
                        [&](int i, int cc, float v) { p.h[(size_t)i * D + cc] = v; });
    cur = t.last_open ? t.last : t.last + 1;
    par = 1 - par;
    __syncthreads();
  }
  for (int idx = tid; idx < (ib - cur) * D; idx += kCfThreads)
    p.h[(size_t)cur * D + idx] = 0.f;
  };
  if (rpl == ib - ia + 1) tiles(std::true_type{});
  else tiles(std::false_type{});
}

// ------------------------------------------------------------------ backward
template <int D, int KP, bool BF16>
__global__ __launch_bounds__(kCfThreads, 1) void k_cf_bwd(CfParams p) {
  constexpr int TM = CfShape<D>::TM, NCB = D / 32, SQ = D + 4, SW = D + 4, SH = D + 8;
  constexpr int SA = BF16 ? KP + 8 : KP + 4;
  constexpr int TPR = kCfThreads / TM;   // threads per row in the feature sums
  extern __shared__ __align__(16) unsigned char lds[];
  const CfLds L = cf_plan(D, KP, BF16, true);
  float* abuf = reinterpret_cast<float*>(lds + L.abuf);
  __bf16* hbuf = reinterpret_cast<__bf16*>(lds + L.hbuf);
  float* geo = reinterpret_cast<float*>(lds + L.geo);
  const int* geoi = reinterpret_cast<const int*>(geo);
  int32_t* rps = reinterpret_cast<int32_t*>(lds + L.rp);
  float* qcarry = reinterpret_cast<float*>(lds + L.carry);   // [2][D]
  float* fcarry = qcarry + 2 * D;                            // [2][4]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, li = lane & 31;
  const int cb = wave % NCB, r0 = 32 * (wave / NCB), c = cb * 32 + li;
  const uint32_t N = (uint32_t)p.n_atoms;
  const __amdgpu_buffer_rsrc_t rcol = rsrc(p.col, (uint32_t)p.rowptr[p.n_atoms] * 4u);
  const __amdgpu_buffer_rsrc_t rpos = rsrc(p.pos, N * 12u);
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, N * (uint32_t)D * 4u);
  const __amdgpu_buffer_rsrc_t rgh = rsrc(p.gh, N * (uint32_t)D * 4u);

  stage_weights<D, KP, BF16, true>(p, lds, L);
  const float bias1 = p.cf1[c], bias2 = p.cf2[c];
  const int ia = p.wg_start[blockIdx.x], ib = p.wg_start[blockIdx.x + 1];
  const int rpl = min(ib - ia + 1, kRpMax);
  for (int k = tid; k < rpl; k += kCfThreads) rps[k] = p.rowptr[ia + k];
  for (int k = tid; k < 2 * D + 8; k += kCfThreads) qcarry[k] = 0.f;
  const bool want_gx = p.gx_out != nullptr;
  __syncthreads();
  auto tiles = [&](auto full) {
  const RowPtr<decltype(full)::value> RP{p.rowptr, rps, ia, rpl};
  const int e_begin = RP(ia), e_end = RP(ib);
  int cur = ia, par = 0;
  GeoPrefetch pf{};
  if (tid < TM) pf_start<TM>(pf, RP, ia, e_begin, e_end, rcol, rpos);

  for (int ts = e_begin; ts < e_end; ts += TM) {
    const int te = min(ts + TM, e_end);
    if (tid < TM) {
      tile_geometry<TM, true>(p, pf, geo, ts, te, cur);
      pf_advance<TM>(pf, RP, ts + TM, e_end, rcol, rpos);
    }
    __syncthreads();
    // sender rows, needed after the filter: issue the gathers now
    float xg[16], gg[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t oj = ((uint32_t)geoi[G_J * TM + out_row(r0, r, h)] * D + c) * 4u;
      xg[r] = bload(rx, oj);
      gg[r] = bload(rgh, oj);
    }
    // b~ and d b~ / dd
    for (int idx = tid; idx < TM * KP; idx += kCfThreads) {
      const int r = idx / KP, k = idx - r * KP;
      float bt = 0.f, btp = 0.f;
      if (k < p.Dr && geoi[G_IN * TM + r]) {
        const float z = geo[G_D * TM + r] - (p.rbf_min + (float)k * p.rbf_step);
        const float g = __builtin_amdgcn_exp2f(p.rbf_coef2 * z * z);
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
    __syncthreads();
    // GEMM1 on both operands: a = b~ Wf1, v = (d b~/dd) Wf1
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    if constexpr (BF16) {
      const __bf16* Ap[2] = {hbuf + (r0 + li) * SA + 8 * h, hbuf + (TM + r0 + li) * SA + 8 * h};
      mma_bf16<2, KP>(acc, Ap, reinterpret_cast<const __bf16*>(lds + L.w1), SA, cb * 32, lane);
    } else {
      const float* Ap[2] = {abuf + (r0 + li) * SA + 4 * h, abuf + (TM + r0 + li) * SA + 4 * h};
      mma_f32<2, false, KP>(acc, Ap, reinterpret_cast<const float*>(lds + L.w1), SW, cb * 32, lane);
    }
    __syncthreads();
    // s = ssp(a) -> LDS; keep sigmoid(a) in acc[0] and v in acc[1]
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = out_row(r0, r, h);
      float s, sg;
      ssp_sig(acc[0][r] + bias1, s, sg);
      acc[0][r] = sg;
      if constexpr (BF16) hbuf[row * SH + c] = (__bf16)s;
      else abuf[row * SQ + c] = s;
    }
    __syncthreads();
    f32x16 accw[1] = {f32x16{}};
    if constexpr (BF16) {
      const __bf16* Ap[1] = {hbuf + (r0 + li) * SH + 8 * h};
      mma_bf16<1, D>(accw, Ap, reinterpret_cast<const __bf16*>(lds + L.w2), SH, cb * 32, lane);
    } else {
      const float* Ap[1] = {abuf + (r0 + li) * SQ + 4 * h};
      mma_f32<1, false, D>(accw, Ap, reinterpret_cast<const float*>(lds + L.w2), SW, cb * 32, lane);
    }
    // gathers; q = dE/dh_j * w (source sum), g_w = dE/dh_i * x_j + dE/dh_j * x_i (both directions)
    // receiver rows: all 32 loads are issued before any is used (masks are
    // arithmetic, so no load sits behind a branch)
    float gw[16], xr[16], gr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t oi = ((uint32_t)geoi[G_I * TM + out_row(r0, r, h)] * D + c) * 4u;
      xr[r] = bload(rx, oi);
      gr[r] = bload(rgh, oi);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float mk = geoi[G_IN * TM + out_row(r0, r, h)] ? 1.f : 0.f;
      const float w = mk * (accw[0][r] + bias2);
      accw[0][r] = gg[r] * w;
      gw[r] = mk * (gr[r] * xg[r] + gg[r] * xr[r]);
    }
    __syncthreads();
    const TileSegs t = tile_segs<TM>(RP, geoi, ts, te, cur);
    if (want_gx) {
#pragma unroll
      for (int r = 0; r < 16; ++r) abuf[out_row(r0, r, h) * SQ + c] = accw[0][r];
      __syncthreads();
      seg_sum_cols<D, SQ>(RP, t, ts, te, abuf, qcarry + par * D, qcarry + (1 - par) * D,
                          [&](int i, int cc, float v) {
                            const size_t o = (size_t)i * D + cc;
                            p.gx_out[o] = p.gx_in[o] + v;
                          });
      __syncthreads();
    }
    // g_w -> LDS, GEMM3: g_s = g_w Wf2^T
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = out_row(r0, r, h);
      if constexpr (BF16) hbuf[row * SH + c] = (__bf16)gw[r];
      else abuf[row * SQ + c] = gw[r];
    }
    __syncthreads();
    f32x16 accg[1] = {f32x16{}};
    if constexpr (BF16) {
      const __bf16* Ap[1] = {hbuf + (r0 + li) * SH + 8 * h};
      mma_bf16<1, D>(accg, Ap, reinterpret_cast<const __bf16*>(lds + L.w2n), SH, cb * 32, lane);
    } else {
      const float* Ap[1] = {abuf + (r0 + li) * SQ + 4 * h};
      mma_f32<1, true, D>(accg, Ap, reinterpret_cast<const float*>(lds + L.w2), SW, cb * 32, lane);
    }
    __syncthreads();
    // p = g_s * sigmoid(a) * v, summed over features per edge -> dE/dd
#pragma unroll
    for (int r = 0; r < 16; ++r)
      abuf[out_row(r0, r, h) * SQ + c] = accg[0][r] * acc[0][r] * acc[1][r];
    __syncthreads();
    {
      const int r = tid / TPR, part = tid - r * TPR;
      float s = 0.f;
      const float* rowp = abuf + r * SQ + part * (D / TPR);
#pragma unroll
      for (int k = 0; k < D / TPR; ++k) s += rowp[k];
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) s += __shfl_xor(s, o, 64);
      if (part == 0) {
        const float gd = geoi[G_IN * TM + r] ? s * geo[G_INVD * TM + r] : 0.f;
        geo[G_FX * TM + r] = gd * geo[G_UX * TM + r];
        geo[G_FY * TM + r] = gd * geo[G_UY * TM + r];
        geo[G_FZ * TM + r] = gd * geo[G_UZ * TM + r];
      }
    }
    __syncthreads();
    // force rows: one thread per (receiver, component)
    {
      float* fin = fcarry + par * 4;
      float* fout = fcarry + (1 - par) * 4;
      const int comp = tid & 3;
      for (int k = tid >> 2; k < t.nseg && comp < 3; k += kCfThreads / 4) {
        const int i = t.first + k;
        const int rs = RP(i), re = RP(i + 1);
        const int lo = (rs > ts ? rs : ts) - ts, hi = (re < te ? re : te) - ts;
        float s = 0.f;
        for (int r = lo; r < hi; ++r) s += geo[(G_FX + comp) * TM + r];
        if (k == 0) s += fin[comp];
        if (k == t.nseg - 1) {
          if (t.last_open) {
            fout[comp] = s;
            continue;
          }
          fout[comp] = 0.f;
        }
        float* f = p.forces + (size_t)i * 3 + comp;
        *f = (p.force_accumulate ? *f : 0.f) - s;
      }
    }
    cur = t.last_open ? t.last : t.last + 1;
    par = 1 - par;
    __syncthreads();
  }
  for (int idx = tid; idx < (ib - cur) * D; idx += kCfThreads) {
    const size_t o = (size_t)cur * D + idx;
    if (want_gx) p.gx_out[o] = p.gx_in[o];
  }
  if (!p.force_accumulate)
    for (int idx = tid; idx < (ib - cur) * 3; idx += kCfThreads) p.forces[(size_t)cur * 3 + idx] = 0.f;
  };
  if (rpl == ib - ia + 1) tiles(std::true_type{});
  else tiles(std::false_type{});
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

// ------------------------------------------------------------------ dispatch
template <int D, int KP, bool BF16>
static hipError_t set_lds_limit_one() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_cf_fwd<D, KP, BF16>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_cf_bwd<D, KP, BF16>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

template <template <int, int, bool> class Fn>
static hipError_t cf_dispatch(int D, int KP, int bf16, typename Fn<64, 32, false>::Arg a) {
#define SN_CF(DD, KK, BB) if (D == DD && KP == KK && (bf16 != 0) == BB) return Fn<DD, KK, BB>::run(a);
  SN_CF(64, 32, false) SN_CF(64, 56, false) SN_CF(64, 64, false)
  SN_CF(128, 32, false) SN_CF(128, 56, false) SN_CF(128, 64, false)
  SN_CF(64, 32, true) SN_CF(64, 64, true) SN_CF(128, 32, true) SN_CF(128, 64, true)
#undef SN_CF
  return hipErrorInvalidValue;
}

struct LaunchArg { const CfParams* p; int G; hipStream_t s; };
template <int D, int KP, bool BF16> struct PrepFn {
  using Arg = int;
  static hipError_t run(int) { return set_lds_limit_one<D, KP, BF16>(); }
};
template <int D, int KP, bool BF16> struct FwdFn {
  using Arg = LaunchArg;
  static hipError_t run(LaunchArg a) {
    hipLaunchKernelGGL((k_cf_fwd<D, KP, BF16>), dim3(a.G), dim3(kCfThreads),
                       cf_lds_bytes(D, KP, BF16, 0), a.s, *a.p);
    return hipGetLastError();
  }
};
template <int D, int KP, bool BF16> struct BwdFn {
  using Arg = LaunchArg;
  static hipError_t run(LaunchArg a) {
    hipLaunchKernelGGL((k_cf_bwd<D, KP, BF16>), dim3(a.G), dim3(kCfThreads),
                       cf_lds_bytes(D, KP, BF16, 1), a.s, *a.p);
    return hipGetLastError();
  }
};

hipError_t cf_prepare(int D, int KP, int bf16) { return cf_dispatch<PrepFn>(D, KP, bf16, 0); }

hipError_t launch_cf_forward(int D, int bf16, const CfParams& p, int G, hipStream_t s) {
  return cf_dispatch<FwdFn>(D, p.KP, bf16, LaunchArg{&p, G, s});
}

hipError_t launch_cf_backward(int D, int bf16, const CfParams& p, int G, hipStream_t s) {
  return cf_dispatch<BwdFn>(D, p.KP, bf16, LaunchArg{&p, G, s});
}

} // namespace sn
