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
// Work decomposition. Every wave is an independent worker: a work-group
// copies the filter weights into LDS once, which is its only barrier; then
// each of its waves walks its own contiguous range of edges in tiles of 16
// (k_setup gives every worker the same number of whole tiles, to one).
// A receiver whose edges a worker boundary cuts is written by the worker
// holding its last edge; the earlier workers leave their parts in side
// buffers, which the kernels that next read the output add in worker order
// (no atomics; fixed order; cut_workers names the workers from the row
// pointers alone).
//
// Edge-on-lane products. Every product is computed transposed,
// OUT^T[n][e] = sum_k W^T[n][k] IN^T[k][e], on 16x16 MFMA blocks: the weights
// (rows n) are the A operand, read from LDS, and the per-edge activations the
// B operand, one edge per lane column (lane = e + 16 g; the four lane groups g
// hold different feature rows). The accumulator layout of one product (lane
// group g holds features 4g..4g+3 of each 16-feature block) is then exactly
// the B-operand layout of the next, so basis -> GEMM1 -> shifted softplus ->
// GEMM2 never leaves registers. The k index inside each MFMA is permuted to
// match the rows a lane holds, and the weight images in LDS are laid out
// (XOR-swizzled, permuted for 16-bit types) so that every A operand is one 8- or
// 16-byte read. Each lane computes its own edge's geometry and basis and
// gathers its own sender/receiver feature rows with 16-byte loads.
//
// Aggregation. The per-receiver sum runs over edges, i.e. across lanes: 64
// features of messages at a time are transposed through a 4 KiB per-wave LDS
// tile so that every lane holds one feature for the tile's 16 edges, and a
// segmented scan down that column yields each receiver's sum. A receiver still
// open at the tile's end carries its partial sum into the next tile. The
// segment ends of the next 64 receivers come from one lane-parallel load per
// tile. The three force components of the backward are summed the same way
// but without the transpose: each edge's lane already holds them, and a
// segmented scan along the 16-lane rows (row shifts of the cross-lane data
// path) leaves each receiver's total at its last edge's lane. Nothing
// edge-sized reaches HBM and every output row has one writer.
//
// Backward (forces). The neighbour list is symmetric and w_ij = w_ji, so the
// owner of receiver i produces, from its own row alone,
//   q_i       = sum_j dE/dh_j * w_ij         (source sum; the residual
//                                            dE/dx' is added by the next
//                                            atom-wise kernel)
//   dE/dd_ij  = <dE/dw_ij, dw_ij/dd>,  dE/dw_ij = dE/dh_i * x_j + dE/dh_j * x_i
//   dE/dr_i   = sum_j dE/dd_ij (r_i - r_j) / d_ij
// dw/dd is carried forward through the recomputed filter (forward-mode along
// the single scalar d): a' = (d b~/dd) Wf1, s' = sigmoid(a) a', w' = s' Wf2.
// The tangents go through the same products as the values (same weight
// images), so the backward needs no transposed product and lands dE/dd on the
// edge's own lanes. Each interaction block writes its own force rows; a small
// kernel sums the blocks.
//
// Base-2 units (every precision but the fp16 pairs): the basis enters the
// first product multiplied by log2 e, and both biases are stored multiplied by
// log2 e, so that the first product yields u = a log2 e, the shifted softplus
// is taken as ssp(a) / ln 2 = max(u, 0) + log2((1 + 2^-|u|) / 2) (no multiply
// by log2 e or ln 2 per value), and the second product, starting from its
// bias, yields w log2 e. The sums over a receiver's edges (h, q) and dE/dd
// are scaled back by ln 2 once each, where they leave the kernel; the biases
// are the accumulators' starting values, so no per-value bias add remains.
//
// MFMA: v_mfma_f32_16x16x4_f32 (fp32 filters), v_mfma_f32_16x16x32_bf16
// (bfloat16 filters) or v_mfma_f32_16x16x32_f16 (fp16 filters whose weight
// columns carry power-of-two scales, §4.4 "Channel-wise quantization"), fp32
// accumulation throughout.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>

#include "tile16.hpp"

namespace sn {

constexpr int kEdges = 16;  // edges per wave tile: the MFMA column dimension
// Byte offset of a feature row that lies past the end of every per-atom array
// (the library admits at most 2^22 atoms, so N D 4 <= 2^31, and the offsets
// added to it stay below 2^31 + 512): bounded buffer loads from it read zeros.
constexpr uint32_t kMaskedRow = 0x80000000u;

// The filter runs in base-2 units (above) in every precision but the fp16
// pairs, whose operand scales are bounds of the unscaled basis and softplus.
template <int PR>
constexpr bool kBase2 = PR != PREC_F16X2;
// Accumulators start from the bias where no column scale follows the product.
template <int PR>
constexpr bool kBiasInit = PR == PREC_F32 || PR == PREC_BF16;
// The kernels request their first gathers before the first product with the
// 16-bit filters (faster there); at fp32 and on fp16 pairs the backward would
// spill and the forward runs no faster, so they request them after it.
template <int PR>
constexpr bool kEarlyGather = PR == PREC_BF16 || PR == PREC_F16S;
// Weight reads of the second product scheduled ahead of their products
// (pipeline_gemm2_reads) with bf16 filters, where the compiler otherwise
// makes each product wait on its own read (measured: backward 1-3 % faster;
// fp32 unchanged).
template <int PR>
constexpr bool kPipelineReads = PR == PREC_BF16;
// A sum over messages (h, q) or a dE/dd leaving the kernel, back in natural units.
template <int PR>
__device__ __forceinline__ float out_scale(float v) {
  return kBase2<PR> ? v * LN2F : v;
}

__device__ __forceinline__ float min_image(float u, float box, float half) {
  if (u > half) return u - box;
  if (u < -half) return u + box;
  return u;
}

// ------------------------------------------------------------------ LDS plan
// Weight image (built on the host, copied verbatim) then one transpose tile per wave.
//   W1  : Wf1^T [D][KP] (k zero-padded past Dr); fp16 pairs: the hi image,
//         then the lo image (W1L)
//   W2  : Wf2^T [D][D] (16-bit: positions permuted by perm32); fp16 pairs:
//         hi, then lo (W2L)
//   BIAS: cf1[D], cf2[D] (fp32); then, for fp16 filters, the column scales
//         s1[D], s2[D], or for fp16 pairs the split scales (SplitScales);
//         staged only where LDS has room, else read from the image in
//         global memory
// Rows are output-major: the A operand of a lane is a run of its row.
template <int D, int KP, int PR, int NW_>
struct Plan {
  static constexpr int NW = NW_;               // workers (waves) per work-group
  static constexpr int NT = NW * 64;
  static constexpr int ES = PR != PREC_F32 ? 2 : 4;
  static constexpr int NS = PR == PREC_F16X2 ? 2 : 1;   // images per matrix
  static constexpr int W1 = 0;
  static constexpr int W1L = W1 + D * KP * ES;
  static constexpr int W2 = W1 + NS * D * KP * ES;
  static constexpr int W2L = W2 + D * D * ES;
  static constexpr int BIAS = W2 + NS * D * D * ES;
  static constexpr int SC = BIAS + 2 * D * 4;
  static constexpr int IMG = SC + (PR == PREC_F16S ? 2 * D * 4 : PR == PREC_F16X2 ? 32 : 0);
  static constexpr int TB = kEdges * 64 * 4;   // transpose tile: 64 columns of 16 rows
  static constexpr int LDS_MAX = 160 * 1024;
  static constexpr bool BIAS_LDS = IMG + NW * TB <= LDS_MAX;
  static constexpr int STAGE = BIAS_LDS ? IMG : BIAS;   // bytes copied into LDS
  static constexpr int TOTAL = STAGE + NW * TB;
  static_assert(IMG % 16 == 0 && STAGE % 16 == 0, "image is copied in 16-byte pieces");
  static_assert(TOTAL <= LDS_MAX, "LDS plan exceeds 160 KiB");
};

// Waves per work-group of each kernel at one work-group per CU: the forward
// fits 128 registers (four waves per SIMD); the backward needs up to 256 at
// D = 128 (two per SIMD; at three it spills and runs slower).
template <int D, int PR, bool BWD>
constexpr int cf_nw() {
  return BWD ? 8 : 16;
}
// The first block's backward (no source sums) fits 168 registers: three waves
// per SIMD.
template <int D, int PR>
constexpr int cf_nw_first() {
  return 12;
}

int cf_kp(int Dr, int prec) {
  (void)prec;
  return Dr <= 32 ? 32 : 64;
}
int cf_chunks(int Dr, int prec) { return prec != PREC_F32 ? (Dr + 31) / 32 : (Dr + 7) / 8; }

// Scales of the fp16-pair filter (8 floats at Plan::SC). Product q's input
// is multiplied by a[q] before it is split, its weights by a power of two
// sw, and its output by u[q] = 1 / (sw a[q]); q = 0: basis into Wf1, 1: basis
// derivative into Wf1, 2: softplus output into Wf2, 3: its tangent into Wf2.
struct SplitScales {
  float a[4], u[4];
};

// v = m 2^e with m in [0.5, 1): e (0 for v = 0)
static int binade(double v) {
  int e = 0;
  if (v > 0) std::frexp(v, &e);
  return e;
}

// fp16-pair images and scales. Each matrix is scaled by the power of two
// that puts its largest magnitude in [2^13, 2^14), then stored as fp16 hi
// and lo images. The product inputs get powers of two that map a bound of
// their magnitude into [2^12, 2^13), far inside fp16's range (65504):
//   basis          b~_k = g_k C <= 1
//   its derivative |d b~_k/dd| <= e^(-1/2) / sigma + pi / (2 r_c)   (=: B1;
//                  the Gaussian's slope peaks at d - mu_k = sigma, and
//                  |C'| <= pi / (2 r_c), |C|, g_k <= 1)
//   softplus out   |ssp(a_n)| <= max(|a_n|, ln 2), |a_n| <= A_n + |cf1_n|
//                  with A_n = sum_k |Wf1[k][n]| (the basis is in [0, 1])
//   its tangent    |sigmoid(a_n) a'_n| <= A_n B1
// Exponents are clamped so that every scale and u stays a normal float.
template <int D, int KP>
static void fill_split(int Dr, const float* Wf1, const float* cf1, const float* Wf2,
                       float rbf_step, float r_cut, unsigned char* w1h, unsigned char* w1l,
                       unsigned char* w2h, unsigned char* w2l, SplitScales& sc) {
  auto w1 = [&](int k, int n) { return Wf1[(size_t)k * D + n]; };
  auto w2 = [&](int k, int n) { return Wf2[(size_t)k * D + n]; };
  double m1 = 0, m2 = 0, Amax = 0, B2 = std::log(2.0);
  for (int n = 0; n < D; ++n) {
    double An = 0;
    for (int k = 0; k < Dr; ++k) {
      An += std::fabs((double)w1(k, n));
      m1 = std::fmax(m1, std::fabs((double)w1(k, n)));
    }
    Amax = std::fmax(Amax, An);
    B2 = std::fmax(B2, An + std::fabs((double)cf1[n]));
    for (int k = 0; k < D; ++k) m2 = std::fmax(m2, std::fabs((double)w2(k, n)));
  }
  const double B1 = std::exp(-0.5) / (double)rbf_step + M_PI / (2.0 * (double)r_cut);
  const double B[4] = {1.0, B1, B2, Amax * B1};
  const int e1 = std::max(binade(m1), -100), e2 = std::max(binade(m2), -100);
  const float s1 = std::ldexp(1.f, 14 - e1), s2 = std::ldexp(1.f, 14 - e2);
  for (int q = 0; q < 4; ++q) {
    const int ew = q < 2 ? e1 : e2;
    const int eb = std::max(binade(B[q]), -99 - ew);   // u = 2^(ew + eb - 27) >= 2^-126
    sc.a[q] = std::ldexp(1.f, 13 - eb);
    sc.u[q] = std::ldexp(1.f, ew + eb - 27);
  }
  auto hi = [](float v) { return (float)(_Float16)v; };
  om_image<KP, PREC_F16S, false>(D, Dr, D, [&](int k, int n) { return hi(w1(k, n) * s1); }, w1h,
                                 nullptr);
  om_image<KP, PREC_F16S, false>(
      D, Dr, D, [&](int k, int n) { const float v = w1(k, n) * s1; return v - hi(v); }, w1l,
      nullptr);
  om_image<D, PREC_F16S, true>(D, D, D, [&](int k, int n) { return hi(w2(k, n) * s2); }, w2h,
                               nullptr);
  om_image<D, PREC_F16S, true>(
      D, D, D, [&](int k, int n) { const float v = w2(k, n) * s2; return v - hi(v); }, w2l,
      nullptr);
}

// Wf1 without the perm32 placement: the first product's B operand (the
// basis) is evaluated directly in the k order a lane feeds.
template <int D, int KP, int PR>
static void fill_image(int Dr, const float* Wf1, const float* cf1, const float* Wf2,
                       const float* cf2, float rbf_step, float r_cut, unsigned char* out) {
  using P = Plan<D, KP, PR, 1>;
  std::memset(out, 0, P::IMG);
  float* sc = reinterpret_cast<float*>(out + P::SC);
  if constexpr (PR == PREC_F16X2) {
    SplitScales ss;
    fill_split<D, KP>(Dr, Wf1, cf1, Wf2, rbf_step, r_cut, out + P::W1, out + P::W1L, out + P::W2,
                      out + P::W2L, ss);
    std::memcpy(sc, &ss, sizeof(ss));
  } else {
    om_image<KP, PR, false>(D, Dr, D, [&](int k, int n) { return Wf1[(size_t)k * D + n]; },
                            out + P::W1, sc);
    om_image<D, PR, true>(D, D, D, [&](int k, int n) { return Wf2[(size_t)k * D + n]; },
                          out + P::W2, sc + D);
  }
  float* bias = reinterpret_cast<float*>(out + P::BIAS);
  const double k = kBase2<PR> ? 1.4426950408889634074 : 1.0;   // log2 e
  for (int n = 0; n < D; ++n) {
    bias[n] = (float)(k * (double)cf1[n]);
    bias[D + n] = (float)(k * (double)cf2[n]);
  }
}

template <class P>
__device__ __forceinline__ void stage_image(const void* img, unsigned char* lds) {
  stage_lds<P::STAGE, P::NT>(img, lds);
}

// cf1 (idx < D) or cf2 (idx - D) values idx .. idx + 3 with idx = lo + k: lo
// is this lane's part (computed inside the tile loop), k a compile-time
// constant folded into the load's offset.
template <class P>
__device__ __forceinline__ f32x4 bias4(const CfParams& p, const unsigned char* lds, int lo, int k) {
  const unsigned char* base =
      P::BIAS_LDS ? lds + P::BIAS : reinterpret_cast<const unsigned char*>(p.img) + P::BIAS;
  return *reinterpret_cast<const f32x4*>(base + 4 * lo + 4 * k);
}
// Column scales s1 (idx < D) or s2 (idx - D), as bias4 (fp16 filters only).
template <class P>
__device__ __forceinline__ f32x4 scale4(const CfParams& p, const unsigned char* lds, int lo, int k) {
  const unsigned char* base =
      P::BIAS_LDS ? lds + P::SC : reinterpret_cast<const unsigned char*>(p.img) + P::SC;
  return *reinterpret_cast<const f32x4*>(base + 4 * lo + 4 * k);
}

// The fp16-pair scales, wave-uniform (scalar loads from the image in global memory).
template <class P>
__device__ __forceinline__ SplitScales split_scales(const CfParams& p) {
  const __attribute__((address_space(4))) float* s =
      (const __attribute__((address_space(4))) float*)(static_cast<const unsigned char*>(p.img) +
                                                       P::SC);
  SplitScales r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r.a[q] = s[q];
    r.u[q] = s[4 + q];
  }
  return r;
}

// ------------------------------------------------------------------ per-edge geometry
struct Geo {
  float d0;            // d - rbf_min
  float C, Cp, in;     // envelope, its d-derivative, 1 inside the cutoff (0 also for padding lanes)
  float invd, ux, uy, uz;
};

__device__ __forceinline__ Geo geometry(const CfParams& p, __amdgpu_buffer_rsrc_t rpos, int recv,
                                        float xj, float yj, float zj, bool valid) {
  const uint32_t oi = (uint32_t)recv * 12u;
  float ux = bload(rpos, oi) - xj;
  float uy = bload(rpos, oi + 4) - yj;
  float uz = bload(rpos, oi + 8) - zj;
  if (p.periodic) {
    ux = min_image(ux, p.box, p.half_box);
    uy = min_image(uy, p.box, p.half_box);
    uz = min_image(uz, p.box, p.half_box);
  }
  // hardware sqrt / rcp (1 ulp) and sin / cos of an angle given in turns,
  // d / (2 r_c) in [0, 1/2] (about 1e-7 absolute)
  const float d = __builtin_amdgcn_sqrtf(ux * ux + uy * uy + uz * uz);
  const float turns = fminf(d, p.r_cut) * p.half_over_rc;
  const float cs = __builtin_amdgcn_cosf(turns), sn = __builtin_amdgcn_sinf(turns);
  Geo g;
  g.d0 = d - p.rbf_min;
  g.in = (valid && d < p.r_cut) ? 1.f : 0.f;
  g.C = 0.5f * (cs + 1.f);
  g.Cp = -0.5f * p.pi_over_rc * sn;
  g.invd = d > 0.f ? __builtin_amdgcn_rcpf(d) : 0.f;
  g.ux = ux; g.uy = uy; g.uz = uz;
  return g;
}

// ------------------------------------------------------------------ products
// Accumulator element r of block nb (lane group g) is feature 16 nb + 4 g + r
// of edge lane % 16.

// GEMM1: acc[q][nb] += sum_k Wf1[k][16 nb + e] * basis_q(k) for k < 8 KC (fp32)
// or 32 KC (16-bit); basis_0 = b~ (Gaussian x envelope), basis_1 = d b~ / dd.
// Each lane evaluates the basis of its own edge for the k slots it feeds
// (fp32: k = 8c + 2g + u for the MFMA pair u; 16-bit: k = 32c + 8g + t).
template <int D, int KP, int PR, int NA>
__device__ __forceinline__ void gemm1_plain(f32x4 (&acc)[NA][D / 16], const unsigned char* lds,
                                            const CfParams& p, const Geo& g, int lane_) {
  constexpr bool H16 = PR != PREC_F32;
  const int lane = opaque(lane_), grp = lane >> 4, e = lane & 15;
  constexpr int CH = H16 ? 32 : 8;     // k per chunk
  constexpr int PL = CH / 4;           // k per lane group per chunk
  float step = p.rbf_step;
  asm volatile("" : "+v"(step));
  const int k0 = PL * grp;
  const float coef2 = p.rbf_coef2, inv_s2 = p.rbf_inv_s2;
  // the envelope and its derivative times log2 e (base-2 units)
  static_assert(kBase2<PR>, "the fp16 pairs take gemm1_split");
  const float gC = g.C * LOG2EF, gCp = g.Cp * LOG2EF;
  // one chunk of basis functions: evaluate, then accumulate its products
  auto chunk = [&](int c) {
    float b[NA][PL];
    if constexpr (H16) {
      // the lane's 8 consecutive centres: one exp for the first Gaussian and
      // one for the ratio of neighbours, g_{k+1} = g_k q_k with q_{k+1} = q_k r
      // (centres one step apart), and the tangent factor
      // C' - (d - mu_k) C / sigma^2, which grows by step C / sigma^2 per k
      const float z = __builtin_fmaf(-(float)(k0 + CH * c), step, g.d0);
      float q = __builtin_amdgcn_exp2f(__builtin_fmaf(p.rbf_qa, z, p.rbf_qb));
      if constexpr (NA == 2) {
        float gk = g.in * __builtin_amdgcn_exp2f(coef2 * z * z);
        float tk = gCp - z * inv_s2 * gC;
        const float dt = step * inv_s2 * gC;
#pragma unroll
        for (int t = 0; t < PL; ++t) {
          b[0][t] = gk * gC;
          b[1][t] = gk * tk;
          tk += dt;
          gk *= q;
          q *= p.rbf_r;
        }
      } else {
        // without the tangent the envelope rides along with the Gaussian
        float gk = g.in * gC * __builtin_amdgcn_exp2f(coef2 * z * z);
#pragma unroll
        for (int t = 0; t < PL; ++t) {
          b[0][t] = gk;
          gk *= q;
          q *= p.rbf_r;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < PL; ++t) {
        // d - mu_k with one rounding (the product k step is exact inside the fma)
        const float z = __builtin_fmaf(-(float)(k0 + CH * c + t), step, g.d0);
        const float gs = g.in * __builtin_amdgcn_exp2f(coef2 * z * z);
        b[0][t] = gs * gC;
        if constexpr (NA == 2) b[1][t] = gs * (gCp - z * inv_s2 * gC);
      }
    }
    if constexpr (H16) {
      using E = typename PrecT<PR>::E;
      using V8 = typename PrecT<PR>::V8;
      const E* W1 = reinterpret_cast<const E*>(lds);
      V8 bq[NA];
#pragma unroll
      for (int q = 0; q < NA; ++q)
#pragma unroll
        for (int t = 0; t < 8; ++t) bq[q][t] = (E)b[q][t];
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        const V8 w = *reinterpret_cast<const V8*>(W1 + sw8<KP>(16 * nb + e, CH * c + PL * grp));
#pragma unroll
        for (int q = 0; q < NA; ++q) acc[q][nb] = mfma16(w, bq[q], acc[q][nb]);
      }
    } else {
      const float* W1 = reinterpret_cast<const float*>(lds);
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        const f32x2 w = *reinterpret_cast<const f32x2*>(W1 + sw4<KP>(16 * nb + e, CH * c + PL * grp));
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int q = 0; q < NA; ++q) acc[q][nb] = mfma16(w[u], b[q][u], acc[q][nb]);
      }
    }
  };
  if constexpr (H16) {
    // the 16-bit layouts always run KP / 32 chunks (p.KC): a compile-time
    // count lets the first chunk's products start from a zero accumulator
    // operand instead of zeroed registers
#pragma unroll
    for (int c = 0; c < KP / 32; ++c) chunk(c);
  } else {
    // the first chunk peeled for the same reason (KC >= 1)
    chunk(0);
#pragma unroll 1
    for (int c = 1; c < p.KC; ++c) chunk(c);
  }
}

// All KP / 32 basis chunks at once (KC = KP / 32 for the 16-bit layouts):
// the basis of the lane's 8 k per chunk, split into fp16 pairs, then, as in
// gemm_split_block, every correction product before the hi*hi products.
template <int D, int KP, int NA>
__device__ __forceinline__ void gemm1_split(f32x4 (&acc)[NA][D / 16], const unsigned char* lds,
                                            const CfParams& p, const Geo& g, int lane_, float sa0,
                                            float sa1) {
  constexpr int NC = KP / 32;
  const int lane = opaque(lane_), grp = lane >> 4, e = lane & 15;
  float step = p.rbf_step;
  asm volatile("" : "+v"(step));
  const float coef2 = p.rbf_coef2;
  const float Ca = g.C * sa0, Cpa = g.Cp * sa1, Cia = p.rbf_inv_s2 * g.C * sa1;
  f16x8 bh[NC][NA], bl[NC][NA];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      // d - mu_k with one rounding, as the fp32 path
      const float z = __builtin_fmaf(-(float)(32 * c + 8 * grp + t), step, g.d0);
      const float gs = g.in * __builtin_amdgcn_exp2f(coef2 * z * z);
      // the hi part is pinned: the lo part must be taken against the very hi
      // that is stored (the compiler may form either from the rounded or the
      // exact product; with one hi, hi + lo represents the value either way)
      float b[NA];
      b[0] = gs * Ca;
      if constexpr (NA == 2) b[1] = gs * (Cpa - z * Cia);
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        const _Float16 h = pinned((_Float16)b[q]);
        bh[c][q][t] = h;
        bl[c][q][t] = (_Float16)(b[q] - (float)h);
      }
    }
  const _Float16* W1H = reinterpret_cast<const _Float16*>(lds);
  const _Float16* W1L = W1H + D * KP;
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    f16x8 wh[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int o = sw8<KP>(16 * nb + e, 32 * c + 8 * grp);
      wh[c] = *reinterpret_cast<const f16x8*>(W1H + o);
      const f16x8 wl = *reinterpret_cast<const f16x8*>(W1L + o);
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        acc[q][nb] = mfma16(wl, bh[c][q], acc[q][nb]);
        acc[q][nb] = mfma16(wh[c], bl[c][q], acc[q][nb]);
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int q = 0; q < NA; ++q) acc[q][nb] = mfma16(wh[c], bh[c][q], acc[q][nb]);
  }
}

// fp16 pairs: basis_q enters scaled by a[q] (sa0, sa1), in fp32 as the
// fp32 path computes it, and is split into hi + lo.
template <int D, int KP, int PR, int NA>
__device__ __forceinline__ void gemm1(f32x4 (&acc)[NA][D / 16], const unsigned char* lds,
                                      const CfParams& p, const Geo& g, int lane, float sa0 = 1.f,
                                      float sa1 = 1.f) {
  if constexpr (PR == PREC_F16X2) gemm1_split<D, KP, NA>(acc, lds, p, g, lane, sa0, sa1);
  else gemm1_plain<D, KP, PR, NA>(acc, lds, p, g, lane);
}

// The second filter product (through Wf2), one output block: B operands in
// the precision's own form, or as fp16 pairs of the inputs scaled by a.
template <int D, int PR>
struct W2Op {
  using T = Operand<D, PR>;
  __device__ __forceinline__ static T make(const f32x4 (&s)[D / 16], float) { return T(s); }
};
template <int D>
struct W2Op<D, PREC_F16X2> {
  using T = SplitOperand<D>;
  __device__ __forceinline__ static T make(const f32x4 (&s)[D / 16], float a) { return T(s, a); }
};
template <class P, int D, int PR, class Op>
__device__ __forceinline__ void gemm2_block(f32x4& acc, const Op& op, const unsigned char* lds,
                                            int nb, const ImgLanes<D, PR>& wl) {
  if constexpr (PR == PREC_F16X2) gemm_split_block<D>(acc, op, lds + P::W2, lds + P::W2L, nb, wl);
  else gemm_om_block<D, PR>(acc, op, lds + P::W2, nb, wl);
}

// Schedule of the weight reads of NB output blocks of the second product
// (each block's bias read first where it starts the accumulator): the reads
// run LEAD ahead of the products that use them, one read per MFMA_PER_READ
// products, instead of each product waiting on the read issued just before
// it. Only the order of the instructions is constrained.
template <int PR, int NBLK, int K>
__device__ __forceinline__ void pipeline_gemm2_reads() {
  constexpr int LEAD = 2;
  constexpr int READS = PR == PREC_F32 ? NBLK * (K / 16) : NBLK * (K / 32);
  constexpr int PER = PR == PREC_F32 ? 4 : 1;
  __builtin_amdgcn_sched_group_barrier(0x100, (kBiasInit<PR> ? NBLK : 0) + LEAD, 0);
#pragma unroll
  for (int i = 0; i < READS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// ------------------------------------------------------------------ receiver segments
// Lane l of a window holds rowptr[cur + 1 + l], the end of receiver cur + l's
// segment; INT_MAX past the worker's last receiver ib - 1.
__device__ __forceinline__ int load_window(__amdgpu_buffer_rsrc_t rrow, int cur, int ib, int lane) {
  const int i = cur + lane;
  const int v = bload_i(rrow, (uint32_t)((i < ib ? i : ib - 1) + 1) * 4u);
  return i < ib ? v : INT_MAX;
}
// End of receiver cur + l (l wave-uniform).
__device__ __forceinline__ int seg_end(const CfParams& p, int win, int cur, int ib, int l) {
  if (l < 64) return __builtin_amdgcn_readlane(win, l);
  return cur + l < ib ? cload(p.rowptr, cur + l + 1) : INT_MAX;
}
// Number of receivers from cur on whose segment ends at or before `bound`.
__device__ __forceinline__ int count_ends(const CfParams& p, int win, int cur, int ib, int bound) {
  int n = __builtin_popcountll(__ballot(win <= bound));
  if (n == 64)
    while (seg_end(p, win, cur, ib, n) <= bound) ++n;
  return n;
}

// Transpose tile of a wave: 64 columns of the tile's 16 rows, column-major.
// Accumulator element r of block b (0..3) of lane group g goes to column
// 16 b + 4 r + g, so that the four lane groups write neighbouring columns;
// reader lane L then holds feature col_feature(L) of the 64. 16-byte chunks
// are XOR-swizzled by column so that 8 neighbouring column reads hit distinct
// banks.
__device__ __forceinline__ int tpos(int col, int row) {
  return col * kEdges + ((((row >> 2) ^ ((col >> 1) & 3)) << 2) | (row & 3));
}
__host__ __device__ __forceinline__ int col_feature(int L) {
  return 16 * (L >> 4) + 4 * (L & 3) + ((L >> 2) & 3);
}
// v of the lane k places lower in the same 16-lane row (0 for the row's
// first k lanes).
__device__ __forceinline__ float row_shr(float v, int k) {
  const int x = __builtin_bit_cast(int, v);
  int y;
  switch (k) {
    case 1: y = __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false); break;
    case 2: y = __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false); break;
    case 4: y = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false); break;
    default: y = __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false); break;
  }
  return __builtin_bit_cast(float, y);
}

// Element offsets, in the transpose tile, of this lane's accumulator
// elements r = 0..3 of block 0; block b adds 256 b (tpos(16 b + c, row) =
// 256 b + tpos(c, row) for c < 16). Built once per tile.
struct TileLanes {
  int off[4];
  __device__ __forceinline__ explicit TileLanes(int lane) {
    const int grp = lane >> 4, e = lane & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) off[r] = tpos(4 * r + grp, e);
  }
};
// Writes accumulator block b (0..3) of the current 64 features.
__device__ __forceinline__ void tile_put(float* Tb, int b, const f32x4& m, const TileLanes& tl) {
#pragma unroll
  for (int r = 0; r < 4; ++r) Tb[256 * b + tl.off[r]] = m[r];
}

// Per-receiver sums of this lane's column of the tile (rows past the tile's
// length hold zeros). Receivers cur .. cur + nfin - 1 end in this tile and are
// written through out(i, total); the open receiver's partial sum is carried.
// A segmented inclusive scan runs down the column (one FMA per row with a
// wave-uniform keep factor that is 0 where a receiver's rows begin); at the
// last row of each finished receiver the running value is its total and is
// written out (receivers without rows in the tile get 0). The summation order
// is the plain sequential one.
template <class Out>
__device__ __forceinline__ void column_segments(const CfParams& p, float* Tb, int win, int cur,
                                                int ib, int nfin, int ts, int len, bool open,
                                                float& carry, int lane_, Out out) {
  const int lane = opaque(lane_);
  uint32_t starts = 0, lasts = 0;
  int prev = 0;
  for (int l = 0; l < nfin; ++l) {
    const int b = seg_end(p, win, cur, ib, l) - ts;
    if (b < kEdges) starts |= 1u << b;
    if (b > prev) lasts |= 1u << (b - 1);
    prev = b;
  }
  const float* col = Tb + lane * kEdges;
  const int sw = (lane >> 1) & 3;
  float run = carry;
  int l = 0;   // next finished receiver (wave-uniform)
#pragma unroll
  for (int u = 0; u < kEdges / 4; ++u) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(col + ((u ^ sw) << 2));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * u + r;
      const float keep = ((starts >> row) & 1u) ? 0.f : 1.f;
      run = fmaf(run, keep, t[r]);
      if ((lasts >> row) & 1u) {
        while (seg_end(p, win, cur, ib, l) - ts <= row) out(cur + l++, 0.f);   // no rows here
        out(cur + l++, run);
      }
    }
  }
  for (; l < nfin; ++l) out(cur + l, 0.f);
  carry = (open && prev < len) ? run : 0.f;
}

// ------------------------------------------------------------------ kernels
// Per-worker state shared by the forward and backward walks: the worker's
// range index, its edges [E0, E1) (whole tiles), its receivers [ia, ib) and
// whether the last of them continues past E1 (tail: its part here goes to
// the side buffers). The first receiver may have started before E0.
struct Walk {
  int rid, ia, ib, E0, E1;
  bool tail;
  __amdgpu_buffer_rsrc_t rrow, rcol, rpos;
};

// Work-groups are dealt to the chip's 8 XCDs in turn (work-group b to XCD
// b mod 8), and each XCD has its own L2. The group that runs on XCD x as its
// k-th takes the range index (x's first) + k, so that every XCD walks one
// contiguous part of the list and its L2 holds the rows that part gathers.
// Only which group runs which range changes: the results do not.
__device__ __forceinline__ int xcd_range_index() {
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  const int q = G >> 3, r = G & 7, x = b & 7;
  return x * q + min(x, r) + (b >> 3);
}

// The four waves a SIMD holds (waves w, w + 4, ... of a work-group; waves
// are placed on the SIMDs in turn) take consecutive ranges, so that each
// SIMD's share of tiles is balanced to one tile.
template <class P>
__device__ __forceinline__ bool worker_range(const CfParams& p, int wave, Walk& w) {
  const uint32_t N = (uint32_t)p.n_atoms;
  w.rid = xcd_range_index() * P::NW + (wave & 3) * (P::NW / 4) + (wave >> 2);
  w.ia = cload(p.wg_start, w.rid);
  const int ia1 = cload(p.wg_start, w.rid + 1);
  w.E0 = cload(p.wg_edge, w.rid);
  w.E1 = cload(p.wg_edge, w.rid + 1);
  // the next worker's first receiver, if it started before E1, is ours too
  w.tail = cload(p.rowptr, ia1) < w.E1;
  w.ib = ia1 + (w.tail ? 1 : 0);
  if (w.ia >= w.ib) return false;
  w.rrow = rsrc(p.rowptr, (N + 1) * 4u);
  w.rcol = rsrc(p.col, (uint32_t)cload(p.rowptr, (int)N) * 4u);
  w.rpos = rsrc(p.pos, N * 12u);
  return true;
}

// Per-tile receiver bookkeeping and edge geometry (both kernels).
struct TileHead {
  int te, len, nfin, ncur, recv, j, win_next;
  Geo g;
};

__device__ __forceinline__ TileHead tile_head(const CfParams& p, const Walk& wk, int ts, int cur,
                                              int win, int& jn, float pjx, float pjy, float pjz,
                                              int lane, int e) {
  TileHead t;
  t.te = min(ts + kEdges, wk.E1);
  t.len = t.te - ts;
  t.nfin = count_ends(p, win, cur, wk.ib, t.te);
  const int nin = count_ends(p, win, cur, wk.ib, t.te - 1);
  int recv = cur;
  for (int l = 0; l < nin; ++l) recv += (ts + e >= seg_end(p, win, cur, wk.ib, l)) ? 1 : 0;
  t.recv = recv;
  t.j = jn;
  t.g = geometry(p, wk.rpos, recv, pjx, pjy, pjz, e < t.len);
  t.ncur = cur + t.nfin;
  t.win_next = load_window(wk.rrow, t.ncur, wk.ib, lane);
  jn = bload_i(wk.rcol, (uint32_t)(ts + kEdges + e) * 4u);
  return t;
}

template <int D, int KP, int PR>
__global__ __launch_bounds__((64 * cf_nw<D, PR, false>()), 1) void k_cf_fwd(CfParams p) {
  using P = Plan<D, KP, PR, cf_nw<D, PR, false>()>;
  constexpr int NB = D / 16;
  extern __shared__ __align__(16) unsigned char lds[];
  stage_image<P>(p.img, lds);
  __syncthreads();

  const int lane = threadIdx.x & 63, e = lane & 15;
  const int wave = uni((int)threadIdx.x >> 6);
  Walk wk;
  if (!worker_range<P>(p, wave, wk)) return;
  const int ib = wk.ib;
  float* Tb = reinterpret_cast<float*>(lds + P::STAGE + wave * P::TB);
  const uint32_t N = (uint32_t)p.n_atoms;
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, N * (uint32_t)D * 4u);
  const int fcol = col_feature(lane);
  SplitScales ss{};
  if constexpr (PR == PREC_F16X2) ss = split_scales<P>(p);

  float carry[NB / 4];
#pragma unroll
  for (int pss = 0; pss < NB / 4; ++pss) carry[pss] = 0.f;
  int cur = wk.ia;
  int win = load_window(wk.rrow, cur, ib, lane);
  int jn = bload_i(wk.rcol, (uint32_t)(wk.E0 + e) * 4u);
  float pjx = bload(wk.rpos, (uint32_t)jn * 12u), pjy = bload(wk.rpos, (uint32_t)jn * 12u + 4),
        pjz = bload(wk.rpos, (uint32_t)jn * 12u + 8);

  for (int ts = wk.E0; ts < wk.E1; ts += kEdges) {
    const TileHead th = tile_head(p, wk, ts, cur, win, jn, pjx, pjy, pjz, lane, e);
    const Geo& g = th.g;
    // per-lane offsets, rebuilt each tile (kept for the whole kernel they would
    // only occupy registers)
    const int lane_t = opaque(lane);
    const int g4 = 4 * (lane_t >> 4);   // this lane's feature offset in a block
    const ImgLanes<D, PR> wl(lane_t);
    const TileLanes tl(lane_t);

    // the sender rows of the first 64 features, requested before the first
    // product (16-bit filters) or the second. Lanes of edges that contribute
    // nothing (at or beyond the cutoff, or past the worker's last edge)
    // gather from an offset past the end of x, which the bounded loads read
    // as zeros: their messages vanish without a mask multiply
    const uint32_t xo = g.in > 0.f ? ((uint32_t)th.j * (uint32_t)D + (uint32_t)g4) * 4u
                                   : kMaskedRow;
    f32x4 xg[4];
    if constexpr (kEarlyGather<PR>) {
#pragma unroll
      for (int b = 0; b < 4; ++b) xg[b] = bload4(rx, xo + (uint32_t)(64 * b));
    }

    // s = ssp(b~ Wf1 + cf1) (base-2 units: s / ln 2 from u = a log2 e)
    f32x4 s[1][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      s[0][nb] = kBiasInit<PR> ? bias4<P>(p, lds, g4, 16 * nb) : f32x4{};
    gemm1<D, KP, PR, 1>(s, lds, p, g, lane, ss.a[0], ss.a[1]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (PR == PREC_F16S) {
        const f32x4 c1 = bias4<P>(p, lds, g4, 16 * nb);
        const f32x4 s1 = scale4<P>(p, lds, g4, 16 * nb);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[0][nb][r] = ssp2(fmaf(s[0][nb][r], s1[r], c1[r]));
      } else if constexpr (PR == PREC_F16X2) {
        const f32x4 c1 = bias4<P>(p, lds, g4, 16 * nb);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[0][nb][r] = ssp(fmaf(s[0][nb][r], ss.u[0], c1[r]));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[0][nb][r] = ssp2(s[0][nb][r]);
      }
    }
    pjx = bload(wk.rpos, (uint32_t)jn * 12u);
    pjy = bload(wk.rpos, (uint32_t)jn * 12u + 4);
    pjz = bload(wk.rpos, (uint32_t)jn * 12u + 8);

    if constexpr (!kEarlyGather<PR>) {
#pragma unroll
      for (int b = 0; b < 4; ++b) xg[b] = bload4(rx, xo + (uint32_t)(64 * b));
    }
    // w = s Wf2 + cf2 (masked beyond the cutoff); messages x_j * w summed per
    // receiver, 64 features at a time; a block's gather registers are
    // refilled with the next 64 features' as soon as they are used
    __builtin_amdgcn_sched_barrier(0);
    // the products of each 64 features are formed right before their
    // messages (fewer live accumulators)
    const auto os = W2Op<D, PR>::make(s[0], ss.a[2]);
#pragma unroll
    for (int pss = 0; pss < NB / 4; ++pss) {
      f32x4 w[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        w[b] = kBiasInit<PR> ? bias4<P>(p, lds, g4, D + 16 * (4 * pss + b)) : f32x4{};
        gemm2_block<P>(w[b], os, lds, 4 * pss + b, wl);
      }
      if constexpr (kPipelineReads<PR>) pipeline_gemm2_reads<PR, 4, D>();
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int nb = 4 * pss + b;
        if constexpr (!kBiasInit<PR>) {
          const f32x4 c2 = bias4<P>(p, lds, g4, D + 16 * nb);
          const f32x4 s2 = PR == PREC_F16S ? scale4<P>(p, lds, g4, D + 16 * nb)
                                           : f32x4{ss.u[2], ss.u[2], ss.u[2], ss.u[2]};
#pragma unroll
          for (int r = 0; r < 4; ++r) w[b][r] = fmaf(w[b][r], s2[r], c2[r]);
        }
        f32x4 m;
#pragma unroll
        for (int r = 0; r < 4; ++r) m[r] = xg[b][r] * w[b][r];
        tile_put(Tb, b, m, tl);
        if (pss + 1 < NB / 4) xg[b] = bload4(rx, xo + (uint32_t)(64 * (nb + 4)));
      }
      wave_sync();
      float* hout = p.h + 64 * pss + fcol;
      column_segments(p, Tb, win, cur, ib, th.nfin, ts, th.len, th.ncur < ib, carry[pss], lane,
                      [&](int i, float tot) { hout[(size_t)i * D] = out_scale<PR>(tot); });
      wave_sync();
    }
    cur = th.ncur;
    win = th.win_next;
  }
  // receivers of the worker left without edges; an open tail receiver
  // (cur = ib - 1) leaves its partial sums to the side buffer
  const int zend = wk.tail ? ib - 1 : ib;
  for (int i = cur; i < zend; ++i)
    for (int c = lane; c < D; c += 64) p.h[(size_t)i * D + c] = 0.f;
  if (wk.tail) {
#pragma unroll
    for (int pss = 0; pss < NB / 4; ++pss)
      p.side_h[(size_t)wk.rid * D + 64 * pss + fcol] = out_scale<PR>(carry[pss]);
  }
}

// Q: the block's source sums q are wanted (every block but the first, whose
// input is the embedding). Without them only the tangents are needed: the
// second product's values, the softplus values and the messages drop out.
template <int D, int KP, int PR, bool Q>
__global__ __launch_bounds__((64 * (Q ? cf_nw<D, PR, true>() : cf_nw_first<D, PR>())), 1)
    void k_cf_bwd(CfParams p) {
  using P = Plan<D, KP, PR, (Q ? cf_nw<D, PR, true>() : cf_nw_first<D, PR>())>;
  constexpr int NB = D / 16;
  extern __shared__ __align__(16) unsigned char lds[];
  stage_image<P>(p.img, lds);
  __syncthreads();

  const int lane = threadIdx.x & 63, e = lane & 15;
  const int wave = uni((int)threadIdx.x >> 6);
  Walk wk;
  if (!worker_range<P>(p, wave, wk)) return;
  const int ib = wk.ib;
  float* Tb = reinterpret_cast<float*>(lds + P::STAGE + wave * P::TB);
  const uint32_t N = (uint32_t)p.n_atoms;
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, N * (uint32_t)D * 4u);
  const __amdgpu_buffer_rsrc_t rgh = rsrc(p.gh, N * (uint32_t)D * 4u);
  // (tested at run time as well: with the branches kept, the fp32 kernel's
  // schedule stays within its registers)
  const bool want_q = Q && p.q_out != nullptr;
  const int fcol = col_feature(lane);
  SplitScales ss{};
  if constexpr (PR == PREC_F16X2) ss = split_scales<P>(p);

  float carry[NB / 4];
#pragma unroll
  for (int pss = 0; pss < NB / 4; ++pss) carry[pss] = 0.f;
  float fcarry[3] = {0.f, 0.f, 0.f};   // open receiver's dE/dr so far
  int cur = wk.ia;
  int win = load_window(wk.rrow, cur, ib, lane);
  int jn = bload_i(wk.rcol, (uint32_t)(wk.E0 + e) * 4u);
  float pjx = bload(wk.rpos, (uint32_t)jn * 12u), pjy = bload(wk.rpos, (uint32_t)jn * 12u + 4),
        pjz = bload(wk.rpos, (uint32_t)jn * 12u + 8);

  for (int ts = wk.E0; ts < wk.E1; ts += kEdges) {
    const TileHead th = tile_head(p, wk, ts, cur, win, jn, pjx, pjy, pjz, lane, e);
    const Geo& g = th.g;
    // per-lane offsets, rebuilt each tile (kept for the whole kernel they would
    // only occupy registers)
    const int lane_t = opaque(lane);
    const int g4 = 4 * (lane_t >> 4);   // this lane's feature offset in a block
    const ImgLanes<D, PR> wl(lane_t);
    const TileLanes tl(lane_t);

    // gathers of the first 64 features (x_j, dE/dh_j, x_i, dE/dh_i); edges
    // that contribute nothing read zeros, as in the forward (their source
    // sums and dE/dd vanish). Issued before the first product where the
    // registers allow (16-bit filters with source sums), else before the
    // second.
    const uint32_t jo = g.in > 0.f ? ((uint32_t)th.j * (uint32_t)D + (uint32_t)g4) * 4u
                                   : kMaskedRow;
    const uint32_t io = g.in > 0.f ? ((uint32_t)th.recv * (uint32_t)D + (uint32_t)g4) * 4u
                                   : kMaskedRow;
    // fp16 pairs hold two blocks' gathers, refilled two blocks ahead
    constexpr int GD = PR == PREC_F16X2 ? 2 : 4;
    f32x4 G[GD][4];
    auto gather = [&](int nb, f32x4 (&Gb)[4]) {
      const uint32_t co = (uint32_t)(64 * nb);
      Gb[0] = bload4(rx, jo + co);
      Gb[1] = bload4(rgh, jo + co);
      Gb[2] = bload4(rx, io + co);
      Gb[3] = bload4(rgh, io + co);
    };
    if constexpr (kEarlyGather<PR> && Q) {
#pragma unroll
      for (int b = 0; b < GD; ++b) gather(b, G[b]);
    }

    // GEMM1: a = b~ Wf1 + cf1 and its tangent a' = (d b~/dd) Wf1;
    // s = ssp(a), s' = sigmoid(a) a' (base-2 units: all three times log2 e)
    f32x4 av[2][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      av[0][nb] = kBiasInit<PR> ? bias4<P>(p, lds, g4, 16 * nb) : f32x4{};
      av[1][nb] = f32x4{};
    }
    gemm1<D, KP, PR, 2>(av, lds, p, g, lane, ss.a[0], ss.a[1]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (PR == PREC_F16S) {
        const f32x4 c1 = bias4<P>(p, lds, g4, 16 * nb);
        const f32x4 s1 = scale4<P>(p, lds, g4, 16 * nb);
#pragma unroll
        for (int r = 0; r < 4; ++r) av[0][nb][r] = fmaf(av[0][nb][r], s1[r], c1[r]);
        av[1][nb] *= s1;
      }
      if constexpr (PR == PREC_F16X2) {
        const f32x4 c1 = bias4<P>(p, lds, g4, 16 * nb);
#pragma unroll
        for (int r = 0; r < 4; ++r) av[0][nb][r] = fmaf(av[0][nb][r], ss.u[0], c1[r]);
        av[1][nb] *= ss.u[1];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float sv, sg;
        if constexpr (kBase2<PR>) ssp2_sig(av[0][nb][r], sv, sg);
        else ssp_sig(av[0][nb][r], sv, sg);
        av[0][nb][r] = sv;
        av[1][nb][r] = sg * av[1][nb][r];
      }
    }
    pjx = bload(wk.rpos, (uint32_t)jn * 12u);
    pjy = bload(wk.rpos, (uint32_t)jn * 12u + 4);
    pjz = bload(wk.rpos, (uint32_t)jn * 12u + 8);

    if constexpr (!(kEarlyGather<PR> && Q)) {
#pragma unroll
      for (int b = 0; b < GD; ++b) gather(b, G[b]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // GEMM2: the tangents of all blocks, w' = s' Wf2, and the values w = s Wf2
    // of the first 64 features, as independent product chains; the values of
    // each further 64 features are formed once the previous ones are used
    const auto os = W2Op<D, PR>::make(av[0], ss.a[2]);   // unused (and dropped) without Q
    // fp16 pairs: the values of all features are formed here, so that the
    // split operand (twice the registers of a 16-bit one) dies before the
    // messages; otherwise the values of each further 64 features are formed
    // once the previous ones are used
    constexpr bool VF = PR == PREC_F16X2;
    f32x4 wt[NB], wv[VF ? NB : 4];
    if constexpr (VF) {
      // values first, then tangents: one split operand live at a time
      if (Q) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          wv[nb] = f32x4{};
          gemm2_block<P>(wv[nb], os, lds, nb, wl);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      const auto ot = W2Op<D, PR>::make(av[1], ss.a[3]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        wt[nb] = f32x4{};
        gemm2_block<P>(wt[nb], ot, lds, nb, wl);
      }
    } else {
      const auto ot = W2Op<D, PR>::make(av[1], ss.a[3]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        wt[nb] = f32x4{};
        gemm2_block<P>(wt[nb], ot, lds, nb, wl);
        if (Q && nb < 4) {
          wv[nb] = kBiasInit<PR> ? bias4<P>(p, lds, g4, D + 16 * nb) : f32x4{};
          gemm2_block<P>(wv[nb], os, lds, nb, wl);
        }
      }
    }

    // per 64 features: q = dE/dh_j w summed per receiver;
    // dE/dd += <dE/dh_i x_j + dE/dh_j x_i, w'>. A block's gather registers
    // are refilled with the next 64 features' as soon as they are used.
    float gdd = 0.f;
#pragma unroll
    for (int pss = 0; pss < NB / 4; ++pss) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int nb = 4 * pss + b;
        const int gs = nb % GD;   // this block's gather slot
        const f32x4 xj = G[gs][0], gj = G[gs][1], xi = G[gs][2], gi = G[gs][3];
        if constexpr (PR == PREC_F16S) {
          const f32x4 s2 = scale4<P>(p, lds, g4, D + 16 * nb);
          if constexpr (Q) {
            const f32x4 c2 = bias4<P>(p, lds, g4, D + 16 * nb);
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[VF ? nb : b][r] = fmaf(wv[VF ? nb : b][r], s2[r], c2[r]);
          }
          wt[nb] *= s2;
        }
        if constexpr (PR == PREC_F16X2) {
          if constexpr (Q) {
            const f32x4 c2 = bias4<P>(p, lds, g4, D + 16 * nb);
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[VF ? nb : b][r] = fmaf(wv[VF ? nb : b][r], ss.u[2], c2[r]);
          }
          wt[nb] *= ss.u[3];
        }
        f32x4 qv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (Q) qv[r] = gj[r] * wv[VF ? nb : b][r];
          gdd = fmaf(gi[r] * xj[r] + gj[r] * xi[r], wt[nb][r], gdd);
        }
        if (want_q) tile_put(Tb, b, qv, tl);
        if (nb + GD < NB) gather(nb + GD, G[gs]);
      }
      if (Q && !VF && pss + 1 < NB / 4) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          wv[b] = kBiasInit<PR> ? bias4<P>(p, lds, g4, D + 16 * (4 * (pss + 1) + b)) : f32x4{};
          gemm2_block<P>(wv[b], os, lds, 4 * (pss + 1) + b, wl);
        }
        if constexpr (kPipelineReads<PR>) pipeline_gemm2_reads<PR, 4, D>();
      }
      if (want_q) {
        wave_sync();
        float* qout = p.q_out + 64 * pss + fcol;
        column_segments(p, Tb, win, cur, ib, th.nfin, ts, th.len, th.ncur < ib, carry[pss], lane,
                        [&](int i, float tot) { qout[(size_t)i * D] = out_scale<PR>(tot); });
        wave_sync();
      }
    }
    gdd += __shfl_xor(gdd, 16, 64);
    gdd += __shfl_xor(gdd, 32, 64);
    const float gd = gdd * (kBase2<PR> ? g.invd * LN2F : g.invd);

    // this block's dE/dr rows: the edge contributions gd u summed per receiver
    // by a segmented scan along the tile's 16 rows (one edge per lane of a
    // 16-lane row); the lane at a finished receiver's last row holds its total
    {
      uint32_t starts = 0, lasts = 0;
      int prev = 0;
      for (int l = 0; l < th.nfin; ++l) {
        const int b = seg_end(p, win, cur, ib, l) - ts;
        if (b < kEdges) starts |= 1u << b;
        if (b > prev) lasts |= 1u << (b - 1);
        else if (lane < 3) p.forces[(size_t)(cur + l) * 3 + lane] = 0.f;   // no edges
        prev = b;
      }
      float f[3] = {gd * g.ux, gd * g.uy, gd * g.uz};
      if (e == 0) {
#pragma unroll
        for (int c = 0; c < 3; ++c) f[c] += fcarry[c];
      }
      const uint32_t sm = starts & ((2u << e) - 1u);          // receiver starts at rows <= e
      const int dist = e - (sm ? 31 - __builtin_clz(sm) : 0);  // rows of this receiver before e
#pragma unroll
      for (int k = 1; k < kEdges; k <<= 1) {
        const float keep = dist >= k ? 1.f : 0.f;
#pragma unroll
        for (int c = 0; c < 3; ++c) f[c] = fmaf(row_shr(f[c], k), keep, f[c]);
      }
      if (lane < kEdges && ((lasts >> e) & 1u)) {
#pragma unroll
        for (int c = 0; c < 3; ++c) p.forces[(size_t)th.recv * 3 + c] = f[c];
      }
      const bool open = th.ncur < ib && prev < th.len;
#pragma unroll
      for (int c = 0; c < 3; ++c)
        fcarry[c] = open ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                        __builtin_bit_cast(int, f[c]), th.len - 1))
                         : 0.f;
    }
    cur = th.ncur;
    win = th.win_next;
  }
  // receivers of the worker left without edges; an open tail receiver
  // (cur = ib - 1) leaves its partial sums to the side buffers
  const int zend = wk.tail ? ib - 1 : ib;
  for (int i = cur; i < zend; ++i) {
    if (want_q)
      for (int c = lane; c < D; c += 64) p.q_out[(size_t)i * D + c] = 0.f;
    if (lane < 3) p.forces[(size_t)i * 3 + lane] = 0.f;
  }
  if (wk.tail) {
    if (want_q) {
#pragma unroll
      for (int pss = 0; pss < NB / 4; ++pss)
        p.side_h[(size_t)wk.rid * D + 64 * pss + fcol] = out_scale<PR>(carry[pss]);
    }
    if (lane < 3)
      p.side_f[(size_t)wk.rid * 3 + lane] = lane == 0 ? fcarry[0] : (lane == 1 ? fcarry[1] : fcarry[2]);
  }
}

// ------------------------------------------------------------------ small kernels
// Worker w takes the edges [wg_edge[w], wg_edge[w + 1]) in whole tiles:
// wg_edge[w] = 16 floor(w T / G) with T = ceil(E / 16) tiles, so every
// worker runs floor(T / G) or ceil(T / G) of them. Its receivers start at the
// one holding edge wg_edge[w] (which may have started in an earlier worker),
// or, where wg_edge[w] falls on a receiver boundary, at the first receiver
// starting there (empty receivers at a boundary belong to the worker that
// starts there). The kernels address the edge list with 32-bit byte offsets:
// a list of kMaxListEdges or more edges is refused through the status word.
constexpr int64_t kMaxListEdges = (int64_t)1 << 30;
__device__ __forceinline__ void partition_one(const int32_t* rowptr, int N, int64_t E, int G, int w,
                                              int32_t* wg_start, int32_t* wg_edge) {
  if (w == G) {
    wg_start[G] = N;
    wg_edge[G] = (int32_t)E;
    return;
  }
  const int64_t T = (E + 15) / 16;
  const int64_t e0 = min((int64_t)16 * (((int64_t)w * T) / G), E);
  int lo = 0, hi = N;   // first r with rowptr[r] >= e0 (rowptr[N] = E >= e0)
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)rowptr[mid] >= e0) hi = mid;
    else lo = mid + 1;
  }
  wg_start[w] = ((int64_t)rowptr[lo] > e0) ? lo - 1 : lo;   // lo >= 1 there
  wg_edge[w] = (int32_t)e0;
}

// Set-up of one evaluation in one launch. The first nbp blocks write the
// kernels' partitions (threads 0..G1 the first, the next G2 + 1 threads the
// second, the next G3 + 1 the third; nbp = 0 when no partition is wanted);
// the next nbe blocks write
// the initial features x[i][:] = Emb[types[i]][:] (FlashSchNet §3.2 "SchNet
// model"), four features per thread; any blocks after them apply the MD
// build mark (BuildMark), one position component per thread.
__global__ __launch_bounds__(kThreads) void k_setup(const int32_t* rowptr, int N, int G1,
                                                    int32_t* wg_start1, int32_t* wg_edge1, int G2,
                                                    int32_t* wg_start2, int32_t* wg_edge2, int G3,
                                                    int32_t* wg_start3, int32_t* wg_edge3, int nbp,
                                                    const int32_t* types, const float* emb,
                                                    int log2D, int n_types, float* x, int nbe,
                                                    BuildMark mark, DevStatus* st) {
  if ((int)blockIdx.x < nbp) {
    const int t = blockIdx.x * kThreads + threadIdx.x;
    const int64_t E = rowptr[N];
    if (t == 0) {
      if (E >= kMaxListEdges) dev_fail(st, SN_ERR_UNSUPPORTED, E);
      st->evaluations += 1;
      st->edges_evaluated += E;
    }
    if (t <= G1) partition_one(rowptr, N, E, G1, t, wg_start1, wg_edge1);
    else if (t <= G1 + 1 + G2) partition_one(rowptr, N, E, G2, t - G1 - 1, wg_start2, wg_edge2);
    else if (t <= G1 + G2 + 2 + G3)
      partition_one(rowptr, N, E, G3, t - G1 - G2 - 2, wg_start3, wg_edge3);
    return;
  }
  if ((int)blockIdx.x >= nbp + nbe) {
    if (mark.gate != nullptr && *mark.gate != mark.gate_val) return;
    const int64_t k = (int64_t)(blockIdx.x - nbp - nbe) * kThreads + threadIdx.x;
    if (k == 0) st->n_rebuilds += 1;
    if (k < 3 * (int64_t)N) mark.pos_at_build[k] = mark.pos[k];
    return;
  }
  const int64_t idx = (int64_t)(blockIdx.x - nbp) * kThreads + threadIdx.x;   // float4 index
  const int log2q = log2D - 2;
  if (idx >= ((int64_t)N << log2q)) return;
  const int64_t i = idx >> log2q;
  const int c4 = (int)(idx & ((1 << log2q) - 1));
  int ty = types[i];
  if (ty < 0 || ty >= n_types) {
    if (c4 == 0) dev_fail(st, SN_ERR_INVALID_ARG, i);
    ty = 0;
  }
  reinterpret_cast<f32x4*>(x)[idx] =
      reinterpret_cast<const f32x4*>(emb)[((int64_t)ty << log2q) + c4];
}

hipError_t launch_setup(const int32_t* rowptr, int n_atoms, int G1, int32_t* wg_start1,
                        int32_t* wg_edge1, int G2, int32_t* wg_start2, int32_t* wg_edge2,
                        int G3, int32_t* wg_start3, int32_t* wg_edge3, const int32_t* types,
                        const float* emb, int D, int n_types, float* x, const BuildMark* mark,
                        DevStatus* st, hipStream_t s) {
  const int nbp = rowptr ? (G1 + 1 + G2 + 1 + G3 + 1 + kThreads - 1) / kThreads : 0;
  const int log2D = D == 128 ? 7 : 6;
  const int64_t n4 = x ? (int64_t)n_atoms * D / 4 : 0;   // no x: the features are kept
  const int nbe = (int)((n4 + kThreads - 1) / kThreads);
  const int nbm = mark ? std::max(1, (int)((3 * (int64_t)n_atoms + kThreads - 1) / kThreads)) : 0;
  const int64_t nb = (int64_t)nbp + nbe + nbm;
  if (nb == 0) return hipSuccess;
  const BuildMark mk = mark ? *mark : BuildMark{};
  hipLaunchKernelGGL(k_setup, dim3((unsigned)nb), dim3(kThreads), 0, s, rowptr, n_atoms, G1,
                     wg_start1, wg_edge1, G2, wg_start2, wg_edge2, G3, wg_start3, wg_edge3, nbp,
                     types, emb, log2D, n_types, x, nbe, mk, st);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dispatch
template <int D, int KP, int PR>
struct CfKernels {
  using PF = Plan<D, KP, PR, cf_nw<D, PR, false>()>;
  using PB = Plan<D, KP, PR, cf_nw<D, PR, true>()>;
  using P0 = Plan<D, KP, PR, cf_nw_first<D, PR>()>;
  static hipError_t prepare() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_cf_fwd<D, KP, PR>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, PF::TOTAL);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_cf_bwd<D, KP, PR, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, PB::TOTAL);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_cf_bwd<D, KP, PR, false>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, P0::TOTAL);
  }
  static size_t image_bytes() { return PF::IMG; }
  static int workers(int kind) { return kind == 2 ? P0::NW : kind == 1 ? PB::NW : PF::NW; }
  static void fill(int Dr, const float* Wf1, const float* cf1, const float* Wf2, const float* cf2,
                   float rbf_step, float r_cut, unsigned char* out) {
    fill_image<D, KP, PR>(Dr, Wf1, cf1, Wf2, cf2, rbf_step, r_cut, out);
  }
  static hipError_t fwd(const CfParams& p, int G, hipStream_t s) {
    hipLaunchKernelGGL((k_cf_fwd<D, KP, PR>), dim3(G), dim3(PF::NT), PF::TOTAL, s, p);
    return hipGetLastError();
  }
  static hipError_t bwd(const CfParams& p, int G, hipStream_t s) {
    if (p.q_out != nullptr)
      hipLaunchKernelGGL((k_cf_bwd<D, KP, PR, true>), dim3(G), dim3(PB::NT), PB::TOTAL, s, p);
    else
      hipLaunchKernelGGL((k_cf_bwd<D, KP, PR, false>), dim3(G), dim3(P0::NT), P0::TOTAL, s, p);
    return hipGetLastError();
  }
};

template <class R, class F>
static R cf_dispatch(int D, int KP, int prec, R fail, F f) {
#define SN_CF(DD, KK, PP) \
  if (D == DD && KP == KK && prec == PP) return f(CfKernels<DD, KK, PP>{});
#define SN_CF_P(PP) SN_CF(64, 32, PP) SN_CF(64, 64, PP) SN_CF(128, 32, PP) SN_CF(128, 64, PP)
  SN_CF_P(PREC_F32) SN_CF_P(PREC_BF16) SN_CF_P(PREC_F16S) SN_CF_P(PREC_F16X2)
#undef SN_CF_P
#undef SN_CF
  return fail;
}

hipError_t cf_prepare(int D, int KP, int prec) {
  return cf_dispatch(D, KP, prec, hipErrorInvalidValue,
                     [](auto k) { return decltype(k)::prepare(); });
}
int cf_workers(int D, int KP, int prec, int kind) {
  return cf_dispatch(D, KP, prec, 0, [&](auto k) { return decltype(k)::workers(kind); });
}
size_t cf_image_bytes(int D, int KP, int prec) {
  return cf_dispatch(D, KP, prec, (size_t)0, [](auto k) { return decltype(k)::image_bytes(); });
}
void cf_fill_image(int D, int KP, int prec, int Dr, const float* Wf1, const float* cf1,
                   const float* Wf2, const float* cf2, float rbf_step, float r_cut,
                   unsigned char* out) {
  cf_dispatch(D, KP, prec, 0, [&](auto k) {
    decltype(k)::fill(Dr, Wf1, cf1, Wf2, cf2, rbf_step, r_cut, out);
    return 0;
  });
}
hipError_t launch_cf_forward(int D, int KP, int prec, const CfParams& p, int G, hipStream_t s) {
  return cf_dispatch(D, KP, prec, hipErrorInvalidValue,
                     [&](auto k) { return decltype(k)::fwd(p, G, s); });
}
hipError_t launch_cf_backward(int D, int KP, int prec, const CfParams& p, int G, hipStream_t s) {
  return cf_dispatch(D, KP, prec, hipErrorInvalidValue,
                     [&](auto k) { return decltype(k)::bwd(p, G, s); });
}

} // namespace sn
