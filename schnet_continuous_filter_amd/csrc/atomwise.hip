// Atom-wise layers: type embedding, update network with residual, readout,
// their gradients, and the per-replica energy sum.
//
// FlashSchNet §3.2 "SchNet model": atom types select the initial features;
// "CFConv message passing and aggregation": a point-wise update network with a
// residual connection follows every aggregation; "Energy readout": a per-atom
// network then a sum. §4.1 "Precision contract": energy accumulation in fp32
// or better (the replica sum here accumulates in double).
//
// Each network is two dense products chained through an activation (or gate).
// A work-group copies both weight matrices into LDS once; its waves then take
// 16-atom tiles in turn. Products are computed transposed on 16x16 MFMA blocks
// (v_mfma_f32_16x16x4_f32), one atom per lane column: the weights are the A
// operand (output-major images built on the host), the atom features the B
// operand, loaded from HBM straight into the accumulator layout (lane group g
// holds features 4g..4g+3 of every 16-feature block) and stored back from it.
// The intermediate activation never leaves registers. With fp16 operands
// (§4.4 "W16A16 mixed precision for MLP submodules") every weight column
// carries a power-of-two scale: outputs of a product are multiplied by their
// column's scale, and products with a transposed matrix (the gradients)
// multiply their inputs by it instead. With an fp32 model whose products run
// on fp16 pairs (PREC_F16X2) each matrix is stored as hi and lo fp16 images
// of its values times one power of two, and each atom's input vector is
// scaled by the power of two that puts its largest magnitude in
// [2^12, 2^13) before it is split into hi + lo; the output is scaled back.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "tile16.hpp"

namespace sn {

constexpr int kAtomNW = 16;   // waves per work-group (four per SIMD)

// Bounded store: an offset past the resource's size writes nothing.
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v) {
  using u32x4 = __attribute__((ext_vector_type(4))) uint32_t;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, 0);
}
constexpr int kAtoms = 16;    // atoms per wave tile

// LDS image of one network: M1 [N1][D] (first product, output-major), M2
// [D][N1] (second product), V1 [N1], V2 [D] (vectors of the mode), and for
// fp16 operands the column scales S1 [N1] of the first network layer and S2
// [D] of the second (readout: S1 only). fp16 pairs: M1 and M2 hold the hi
// images, M1L and M2L the lo images, and S1 the two matrices' inverse scales.
template <int D, int N1, int PR>
struct AtomPlan {
  static constexpr int ES = PR != PREC_F32 ? 2 : 4;
  static constexpr int NS = PR == PREC_F16X2 ? 2 : 1;   // images per matrix
  static constexpr int M1 = 0;
  static constexpr int M1L = M1 + N1 * D * ES;
  static constexpr int M2 = M1 + NS * N1 * D * ES;
  static constexpr int M2L = M2 + D * N1 * ES;
  static constexpr int V1 = M2 + NS * D * N1 * ES;
  static constexpr int V2 = V1 + N1 * 4;
  static constexpr int S1 = V2 + D * 4;
  static constexpr int S2 = S1 + N1 * 4;
  static constexpr int IMG = PR == PREC_F16S ? S2 + D * 4 : PR == PREC_F16X2 ? S1 + 16 : S1;
  static_assert(IMG <= 160 * 1024, "atom-wise image exceeds LDS");
  static_assert(IMG % 16 == 0, "image is copied in 16-byte pieces");
};

// Power-of-two scales of the columns of a row-major [rows][cols] matrix.
static std::vector<float> column_scales(const float* W, int rows, int cols) {
  std::vector<float> s(cols);
  for (int n = 0; n < cols; ++n) {
    float amax = 0.f;
    for (int k = 0; k < rows; ++k) amax = std::fmax(amax, std::fabs(W[(size_t)k * cols + n]));
    s[n] = pow2_scale(amax);
  }
  return s;
}

// Products and vectors of each mode (weights row-major [fan_in][fan_out]):
//   ATOM_UPDATE_FWD  a = h Wu1 + cu1 (stored);  x' = x + ssp(a) Wu2 + cu2
//                    M1 = Wu1^T, M2 = Wu2^T, V1 = cu1, V2 = cu2
//   ATOM_UPDATE_BWD  g_a = (g_x Wu2^T) sigmoid(a);  g_h = g_a Wu1^T
//                    M1 = Wu2, M2 = Wu1
//   ATOM_READOUT     o = x Wo1 + co1;  eps = ssp(o).wo2 + co2;
//                    g_x = (sigmoid(o) wo2) Wo1^T
//                    M1 = Wo1^T, M2 = Wo1, V1 = co1, V2[:N1] = wo2
// Weights are divided by their column scales (all 1 unless fp16) before
// they are placed; the kernels multiply the scales back in.
// fp16-pair images of one matrix: m scaled by the power of two that puts
// its largest magnitude in [2^13, 2^14), as hi and lo images (PERM layout of
// chained products); returns the inverse of that scale.
template <int K, class F>
static float pair_images(int N, F m, unsigned char* hi, unsigned char* lo) {
  float amax = 0.f;
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) amax = std::fmax(amax, std::fabs(m(k, n)));
  int e = 0;
  if (amax > 0.f) std::frexp(amax, &e);
  e = std::max(e, -100);
  const float sc = std::ldexp(1.f, 14 - e);
  auto h = [](float v) { return (float)(_Float16)v; };
  om_image<K, PREC_F16S>(N, K, N, [&](int k, int n) { return h(m(k, n) * sc); }, hi, nullptr);
  om_image<K, PREC_F16S>(N, K, N, [&](int k, int n) { const float v = m(k, n) * sc; return v - h(v); },
                         lo, nullptr);
  return std::ldexp(1.f, e - 14);
}

// The products of each mode as in fill_atom_image, on fp16 pairs; S1 holds
// the inverse scales of M1 and M2.
template <int D, int N1>
static void fill_atom_pairs(int mode, const float* W1, const float* b1, const float* W2,
                            const float* b2, unsigned char* out) {
  using P = AtomPlan<D, N1, PREC_F16X2>;
  float* v1 = reinterpret_cast<float*>(out + P::V1);
  float* v2 = reinterpret_cast<float*>(out + P::V2);
  float* inv = reinterpret_cast<float*>(out + P::S1);
  auto w1 = [&](int k, int n) { return W1[(size_t)k * N1 + n]; };   // k < D, n < N1
  auto w2 = [&](int n, int m) { return W2[(size_t)n * D + m]; };    // n < N1, m < D
  if (mode == ATOM_UPDATE_FWD) {
    inv[0] = pair_images<D>(N1, w1, out + P::M1, out + P::M1L);
    inv[1] = pair_images<N1>(D, w2, out + P::M2, out + P::M2L);
    std::memcpy(v1, b1, N1 * sizeof(float));
    std::memcpy(v2, b2, D * sizeof(float));
  } else if (mode == ATOM_UPDATE_BWD) {
    inv[0] = pair_images<D>(N1, [&](int m, int n) { return w2(n, m); }, out + P::M1, out + P::M1L);
    inv[1] = pair_images<N1>(D, [&](int n, int k) { return w1(k, n); }, out + P::M2, out + P::M2L);
  } else {
    inv[0] = pair_images<D>(N1, w1, out + P::M1, out + P::M1L);
    inv[1] = pair_images<N1>(D, [&](int n, int k) { return w1(k, n); }, out + P::M2, out + P::M2L);
    std::memcpy(v1, b1, N1 * sizeof(float));
    for (int n = 0; n < N1; ++n) v2[n] = W2[n];
  }
}

template <int D, int N1, int PR>
static void fill_atom_image(int mode, const float* W1, const float* b1, const float* W2,
                            const float* b2, unsigned char* out) {
  using P = AtomPlan<D, N1, PR>;
  constexpr bool SC = PR == PREC_F16S;
  std::memset(out, 0, P::IMG);
  if constexpr (PR == PREC_F16X2) {
    fill_atom_pairs<D, N1>(mode, W1, b1, W2, b2, out);
    return;
  }
  float* v1 = reinterpret_cast<float*>(out + P::V1);
  float* v2 = reinterpret_cast<float*>(out + P::V2);
  // s1: columns of W1 [D][N1]; s2: columns of W2 [N1][D] (update) 
  std::vector<float> s1(N1, 1.f), s2(D, 1.f);
  if (SC) {
    s1 = column_scales(W1, D, N1);
    if (mode != ATOM_READOUT) s2 = column_scales(W2, N1, D);
    std::memcpy(out + P::S1, s1.data(), N1 * sizeof(float));
    if (mode != ATOM_READOUT) std::memcpy(out + P::S2, s2.data(), D * sizeof(float));
  }
  auto w1 = [&](int k, int n) { return W1[(size_t)k * N1 + n] / s1[n]; };   // k < D, n < N1
  auto w2 = [&](int n, int m) { return W2[(size_t)n * D + m] / s2[m]; };    // n < N1, m < D
  if (mode == ATOM_UPDATE_FWD || mode == ATOM_READOUT)   // M1[n][k] = W1[k][n]
    om_image<D, PR>(N1, D, N1, w1, out + P::M1, nullptr);
  if (mode == ATOM_UPDATE_FWD) {                         // M2[m][n] = W2[n][m]
    om_image<N1, PR>(D, N1, D, [&](int n, int m) { return w2(n, m); }, out + P::M2, nullptr);
    std::memcpy(v1, b1, N1 * sizeof(float));
    std::memcpy(v2, b2, D * sizeof(float));
  } else if (mode == ATOM_UPDATE_BWD) {
    // M1[n][m] = Wu2[n][m] (contraction over m), M2[k][n] = Wu1[k][n] (over n)
    om_image<D, PR>(N1, D, N1, [&](int m, int n) { return w2(n, m); }, out + P::M1, nullptr);
    om_image<N1, PR>(D, N1, D, [&](int n, int k) { return w1(k, n); }, out + P::M2, nullptr);
  } else {
    // M2[k][n] = Wo1[k][n] (over n); V2 = wo2 [N1], on the fp16 grid of its
    // own scale when the operands are fp16
    om_image<N1, PR>(D, N1, D, [&](int n, int k) { return w1(k, n); }, out + P::M2, nullptr);
    std::memcpy(v1, b1, N1 * sizeof(float));
    for (int n = 0; n < N1; ++n) v2[n] = W2[n];
    if (SC) {
      const float so = column_scales(W2, N1, 1)[0];
      for (int n = 0; n < N1; ++n) v2[n] = (float)(_Float16)(W2[n] / so) * so;
    }
  }
}

// Binade of the largest magnitude of this lane's atom vector (its K values
// are spread over the four lane groups of the atom's column): v = m 2^e with
// m in [0.5, 1); e >= -100 so that 2^(13 - e) stays a normal float.
template <int K>
__device__ __forceinline__ int atom_binade(const f32x4 (&v)[K / 16]) {
  float m = 0.f;
#pragma unroll
  for (int kb = 0; kb < K / 16; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(v[kb][r]));
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  int e = 0;
  (void)frexpf(m, &e);
  return max(e, -100);
}

// out[nb] = sum_k M[16 nb + e][k] in[k] on fp16 pairs: the input scaled into
// [2^12, 2^13) per atom, then the product scaled back by inv_m 2^(e - 13)
// (inv_m: the inverse of the matrix's own scale).
template <int K, int NOUT>
__device__ __forceinline__ void atom_pair_product(f32x4 (&out)[NOUT / 16], const f32x4 (&in)[K / 16],
                                                  const unsigned char* hi, const unsigned char* lo,
                                                  float inv_m, int lane) {
  const int e = atom_binade<K>(in);
  const SplitOperand<K> op(in, ldexpf(1.f, 13 - e));
  const ImgLanes<K, PREC_F16X2> ln(opaque(lane));
  const float back = ldexpf(inv_m, e - 13);
#pragma unroll
  for (int nb = 0; nb < NOUT / 16; ++nb) {
    gemm_split_block<K>(out[nb], op, hi, lo, nb, ln);
    out[nb] *= back;
  }
}

// out[j] = sum_k M[16 (nb0 + j) + e][k] S[k] for the NB output blocks from nb0.
template <int K, int NB, int PR>
__device__ __forceinline__ void gemm_om_blocks(f32x4 (&out)[NB], const f32x4 (&S)[K / 16],
                                               const void* img, int lane, int nb0) {
  const ImgLanes<K, PR> ln(opaque(lane));
  const Operand<K, PR> op(S);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    f32x4 acc = f32x4{};
    gemm_om_block<K, PR>(acc, op, img, nb0 + j, ln);
    out[j] = acc;
  }
}

// Adds to v, which holds the row of atom `atom` that a CFConv launch wrote
// (plus, in the update backward, the row it is summed with), the parts of
// that receiver held by other workers (cut_workers), in worker order.
template <int D>
__device__ __forceinline__ void add_cut_parts(f32x4 (&v)[D / 16], const AtomArgs& g, int atom,
                                              bool ok, int g4) {
  const int64_t E = g.cut_rowptr[g.M];
  int w0 = 0, w1 = 0;
  if (ok) cut_workers(g.cut_rowptr[atom], g.cut_rowptr[atom + 1], (E + 15) / 16, g.cut_G, w0, w1);
  for (int w = w0; w < w1; ++w) {
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
      v[kb] += *reinterpret_cast<const f32x4*>(g.cut_side + (size_t)w * D + g4 + 16 * kb);
  }
}

template <int D, int N1, int MODE, int PR>
__global__ __launch_bounds__(64 * kAtomNW, 1) void k_atom(AtomArgs g) {
  using P = AtomPlan<D, N1, PR>;
  constexpr bool SC = PR == PREC_F16S;
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63, e = lane & 15;
  const int wave = uni((int)threadIdx.x >> 6);
  const int ntiles = (g.M + kAtoms - 1) / kAtoms;
  const uint32_t rows = (uint32_t)g.M;
  const __amdgpu_buffer_rsrc_t rA = rsrc(g.A, rows * D * 4u);
  const __amdgpu_buffer_rsrc_t rA2 = rsrc(g.A2, g.A2 ? rows * D * 4u : 0u);
  const __amdgpu_buffer_rsrc_t rR = rsrc(g.R, g.R ? rows * D * 4u : 0u);
  const __amdgpu_buffer_rsrc_t rS = rsrc(g.S, g.S ? rows * N1 * 4u : 0u);
  // outputs through bounded stores: rows past M are dropped without a branch
  const __amdgpu_buffer_rsrc_t rY = rsrc(g.Y, rows * D * 4u);
  const __amdgpu_buffer_rsrc_t rAo = rsrc(g.Aout, g.Aout ? rows * N1 * 4u : 0u);
  const __amdgpu_buffer_rsrc_t rAs = rsrc(g.Asum, g.Asum ? rows * D * 4u : 0u);
  // a tile's input rows: A (+ A2), every load issued before the first is
  // waited for (a missing A2 and rows past M read 0 through their bounded
  // resources), then the parts of receivers cut by the CFConv launch
  auto fetch = [&](int t, f32x4 (&in)[D / 16]) {
    const int g4 = 4 * (opaque(lane) >> 4);
    const int atom = t * kAtoms + e;
    const uint32_t ro = ((uint32_t)atom * D + (uint32_t)g4) * 4u;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      in[kb] = bload4(rA, ro + 64u * kb);
      if constexpr (MODE == ATOM_UPDATE_BWD) in[kb] += bload4(rA2, ro + 64u * kb);
    }
    if (g.cut_side) add_cut_parts<D>(in, g, atom, atom < g.M, g4);
  };
  // the first tile's rows are fetched while the work-group stages the weights
  int t = (int)blockIdx.x + (int)gridDim.x * wave;
  f32x4 in[D / 16];
  if (t < ntiles) fetch(t, in);
  stage_lds<P::IMG, 64 * kAtomNW>(g.img, lds);
  __syncthreads();

  const float* V1 = reinterpret_cast<const float*>(lds + P::V1);
  const float* V2 = reinterpret_cast<const float*>(lds + P::V2);
  const float* S1 = reinterpret_cast<const float*>(lds + P::S1);
  const float* S2 = reinterpret_cast<const float*>(lds + P::S2);
  auto v4 = [&](const float* v, int i) { return *reinterpret_cast<const f32x4*>(v + i); };

  // tiles interleaved over the work-groups first, so that small systems
  // spread one tile per SIMD over all CUs before any SIMD gets a second
  // (the next tile's rows are fetched at the end of each iteration)
  while (t < ntiles) {
    const int g4 = 4 * (opaque(lane) >> 4);   // this lane's feature offset in a block
    const int atom = t * kAtoms + e;
    const bool ok = atom < g.M;
    const uint32_t ro = ((uint32_t)atom * D + (uint32_t)g4) * 4u;    // D-wide rows
    const uint32_t ro1 = ((uint32_t)atom * N1 + (uint32_t)g4) * 4u;  // N1-wide rows
    // the stored pre-activations, issued with the input rows (with fp16
    // pairs, whose operand split needs those registers, after the product)
    constexpr bool PRE_EARLY = PR != PREC_F16X2;
    f32x4 pre[MODE == ATOM_UPDATE_BWD ? N1 / 16 : 1];
    auto fetch_pre = [&]() {
#pragma unroll
      for (int nb = 0; nb < N1 / 16; ++nb) pre[nb] = bload4(rS, ro1 + 64u * nb);
    };
    if constexpr (MODE == ATOM_UPDATE_BWD && PRE_EARLY) fetch_pre();
    if constexpr (MODE == ATOM_UPDATE_BWD) {
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) bstore4(rAs, ro + 64u * kb, in[kb]);
    }

    if constexpr (SC && MODE == ATOM_UPDATE_BWD) {   // contraction over Wu2's columns
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) in[kb] *= v4(S2, g4 + 16 * kb);
    }
    f32x4 u[N1 / 16];
    if constexpr (PR == PREC_F16X2)
      atom_pair_product<D, N1>(u, in, lds + P::M1, lds + P::M1L, S1[0], lane);
    else
      gemm_om<D, N1, PR>(u, in, lds + P::M1, lane);
    if constexpr (MODE == ATOM_UPDATE_BWD && !PRE_EARLY) fetch_pre();
    float ep = 0.f;
#pragma unroll
    for (int nb = 0; nb < N1 / 16; ++nb) {
      if constexpr (SC && MODE != ATOM_UPDATE_BWD) u[nb] *= v4(S1, g4 + 16 * nb);
      if constexpr (MODE == ATOM_UPDATE_FWD) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(V1 + g4 + 16 * nb);
        const f32x4 a = u[nb] + b;
        bstore4(rAo, ro1 + 64u * nb, a);
#pragma unroll
        for (int r = 0; r < 4; ++r) u[nb][r] = ssp(a[r]);
      } else if constexpr (MODE == ATOM_UPDATE_BWD) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float s, sg;
          ssp_sig(pre[nb][r], s, sg);
          u[nb][r] *= sg;
        }
      } else {
        const f32x4 b = *reinterpret_cast<const f32x4*>(V1 + g4 + 16 * nb);
        const f32x4 w2 = *reinterpret_cast<const f32x4*>(V2 + g4 + 16 * nb);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float s, sg;
          ssp_sig(u[nb][r] + b[r], s, sg);
          ep = fmaf(s, w2[r], ep);
          u[nb][r] = sg * w2[r];
        }
      }
    }
    if constexpr (MODE == ATOM_READOUT) {
      ep += __shfl_xor(ep, 16, 64);
      ep += __shfl_xor(ep, 32, 64);
      if (lane < kAtoms && ok) g.eps[atom] = ep + g.b2s;
    }

    if constexpr (SC && MODE != ATOM_UPDATE_FWD) {   // contraction over W1's columns
#pragma unroll
      for (int nb = 0; nb < N1 / 16; ++nb) u[nb] *= v4(S1, g4 + 16 * nb);
    }
    f32x4 res[MODE == ATOM_UPDATE_FWD ? D / 16 : 1];
    if constexpr (MODE == ATOM_UPDATE_FWD) {
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) res[kb] = bload4(rR, ro + 64u * kb);
    }
    f32x4 y[D / 16];
    if constexpr (PR == PREC_F16X2)
      atom_pair_product<N1, D>(y, u, lds + P::M2, lds + P::M2L, S1[1], lane);
    else
      gemm_om<N1, D, PR>(y, u, lds + P::M2, lane);
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      f32x4 v = y[kb];
      if constexpr (SC && MODE == ATOM_UPDATE_FWD) v *= v4(S2, g4 + 16 * kb);
      if constexpr (MODE == ATOM_UPDATE_FWD)
        v += res[kb] + *reinterpret_cast<const f32x4*>(V2 + g4 + 16 * kb);
      bstore4(rY, ro + 64u * kb, v);
    }
    t += (int)gridDim.x * kAtomNW;
    if (t < ntiles) fetch(t, in);
  }
}

// The same networks for small systems, whose few tiles would leave most
// SIMDs idle or give a few of them a second tile: a group of four waves, one
// per SIMD, takes a 16-atom tile. Member m computes hidden blocks
// [m N1/64, (m + 1) N1/64) of the first product and their activation,
// writes them to the group's LDS exchange tile, and after a work-group
// barrier computes output blocks [m D/64, (m + 1) D/64) of the second
// product from all of them. Only the matrices are staged; the vectors are
// read from the image in global memory. The readout's per-atom energy is
// summed over the four members' parts in member order. fp32 operands only
// (with 16-bit operands each member would still convert or split the whole
// input, and the kernels are bound by that, not by the products).
template <int D, int N1, int MODE, int PR>
struct AtomSplitPlan {
  using P = AtomPlan<D, N1, PR>;
  static constexpr int MAT = P::V1;                  // matrices (staged)
  static constexpr int XB = (N1 / 16) * 64 * 16;     // one group's activation tile
  static constexpr int X = MAT;                      // four exchange tiles
  static constexpr int EP = X + 4 * XB;              // readout: [group][member][atom] parts
  static constexpr int TOTAL = EP + (MODE == ATOM_READOUT ? 4 * 4 * kAtoms * 4 : 0);
  static_assert(MAT % 16 == 0, "image is copied in 16-byte pieces");
  static_assert(TOTAL <= 160 * 1024, "split plan exceeds LDS");
};

template <int D, int N1, int MODE, int PR>
__global__ __launch_bounds__(64 * kAtomNW, 1) void k_atom_split(AtomArgs g) {
  using P = AtomPlan<D, N1, PR>;
  using SP = AtomSplitPlan<D, N1, MODE, PR>;
  static_assert(PR == PREC_F32, "fp32 operands only");
  constexpr int NH = N1 / 64, NO = D / 64;   // blocks per member
  static_assert(NH >= 1 && NO >= 1, "four members need 64-wide layers");
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63, e = lane & 15;
  const int wave = uni((int)threadIdx.x >> 6);
  const int grp = wave >> 2, mem = wave & 3;
  const int ntiles = (g.M + kAtoms - 1) / kAtoms;
  const uint32_t rows = (uint32_t)g.M;
  const __amdgpu_buffer_rsrc_t rA = rsrc(g.A, rows * D * 4u);
  const __amdgpu_buffer_rsrc_t rA2 = rsrc(g.A2, g.A2 ? rows * D * 4u : 0u);
  const __amdgpu_buffer_rsrc_t rR = rsrc(g.R, g.R ? rows * D * 4u : 0u);
  const __amdgpu_buffer_rsrc_t rS = rsrc(g.S, g.S ? rows * N1 * 4u : 0u);
  // a tile's input rows, as in k_atom (each member reads all of them)
  auto fetch = [&](int t, f32x4 (&in)[D / 16]) {
    const int g4 = 4 * (opaque(lane) >> 4);
    const int atom = t * kAtoms + e;
    const uint32_t ro = ((uint32_t)atom * D + (uint32_t)g4) * 4u;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      in[kb] = bload4(rA, ro + 64u * kb);
      if constexpr (MODE == ATOM_UPDATE_BWD) in[kb] += bload4(rA2, ro + 64u * kb);
    }
    if (g.cut_side) add_cut_parts<D>(in, g, atom, atom < g.M, g4);
  };
  // the first round's rows are fetched while the work-group stages the weights
  f32x4 in[D / 16];
  {
    const int t = (int)blockIdx.x + (int)gridDim.x * grp;
    if (t < ntiles) fetch(t, in);
  }
  stage_lds<SP::MAT, 64 * kAtomNW>(g.img, lds);
  __syncthreads();
  const unsigned char* gimg = reinterpret_cast<const unsigned char*>(g.img);
  const float* V1 = reinterpret_cast<const float*>(gimg + P::V1);
  const float* V2 = reinterpret_cast<const float*>(gimg + P::V2);
  auto v4 = [&](const float* v, int i) { return *reinterpret_cast<const f32x4*>(v + i); };
  f32x4* xch = reinterpret_cast<f32x4*>(lds + SP::X + grp * SP::XB);
  float* epl = reinterpret_cast<float*>(lds + SP::EP) + grp * 4 * kAtoms;
  const int h0 = mem * NH, o0 = mem * NO;   // first hidden / output block of this member

  // every wave runs the same number of rounds (group 0's tiles); a group
  // without a tile in a round still meets both barriers
  // (the next round's rows are fetched at the end of each round)
  for (int t0 = (int)blockIdx.x; t0 < ntiles; t0 += (int)gridDim.x * 4) {
    const int t = t0 + (int)gridDim.x * grp;
    const bool active = t < ntiles;
    const int g4 = 4 * (opaque(lane) >> 4);
    const int atom = t * kAtoms + e;
    const bool ok = active && atom < g.M;
    const uint32_t ro = ((uint32_t)atom * D + (uint32_t)g4) * 4u;
    const uint32_t ro1 = ((uint32_t)atom * N1 + (uint32_t)g4) * 4u;
    // update backward: this member's quarter of A + A2, stored to Asum only
    // after the barrier (Asum may be A, which the other members still read)
    f32x4 sum[MODE == ATOM_UPDATE_BWD ? NO : 1];
    if (active) {
      f32x4 pre[MODE == ATOM_UPDATE_BWD ? NH : 1];
      if constexpr (MODE == ATOM_UPDATE_BWD) {
#pragma unroll
        for (int j = 0; j < NH; ++j) pre[j] = bload4(rS, ro1 + 64u * (h0 + j));
#pragma unroll
        for (int j = 0; j < NO; ++j) sum[j] = in[o0 + j];
      }
      f32x4 u[NH];
      gemm_om_blocks<D, NH, PR>(u, in, lds + P::M1, lane, h0);
      float ep = 0.f;
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const int c = g4 + 16 * (h0 + j);   // this lane's hidden index of block j
        if constexpr (MODE == ATOM_UPDATE_FWD) {
          const f32x4 a = u[j] + v4(V1, c);
          if (ok) *reinterpret_cast<f32x4*>(g.Aout + (size_t)atom * N1 + c) = a;
#pragma unroll
          for (int r = 0; r < 4; ++r) u[j][r] = ssp(a[r]);
        } else if constexpr (MODE == ATOM_UPDATE_BWD) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float sp, sg;
            ssp_sig(pre[j][r], sp, sg);
            u[j][r] *= sg;
          }
        } else {
          const f32x4 b = v4(V1, c);
          const f32x4 w2 = v4(V2, c);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float sp, sg;
            ssp_sig(u[j][r] + b[r], sp, sg);
            ep = fmaf(sp, w2[r], ep);
            u[j][r] = sg * w2[r];
          }
        }
        xch[(h0 + j) * 64 + lane] = u[j];
      }
      if constexpr (MODE == ATOM_READOUT) {
        ep += __shfl_xor(ep, 16, 64);
        ep += __shfl_xor(ep, 32, 64);
        if (lane < kAtoms) epl[mem * kAtoms + lane] = ep;
      }
    }
    __syncthreads();
    if (active) {
      if constexpr (MODE == ATOM_UPDATE_BWD) {
        if (g.Asum && ok) {
#pragma unroll
          for (int j = 0; j < NO; ++j)
            *reinterpret_cast<f32x4*>(g.Asum + (size_t)atom * D + g4 + 16 * (o0 + j)) = sum[j];
        }
      }
      f32x4 uf[N1 / 16];
#pragma unroll
      for (int nb = 0; nb < N1 / 16; ++nb) uf[nb] = xch[nb * 64 + lane];
      if constexpr (MODE == ATOM_READOUT) {
        if (mem == 0 && lane < kAtoms && ok) {
          const float* q = epl + lane;
          g.eps[atom] = ((q[0] + q[kAtoms]) + q[2 * kAtoms]) + q[3 * kAtoms] + g.b2s;
        }
      }
      f32x4 res[MODE == ATOM_UPDATE_FWD ? NO : 1];
      if constexpr (MODE == ATOM_UPDATE_FWD) {
#pragma unroll
        for (int j = 0; j < NO; ++j) res[j] = bload4(rR, ro + 64u * (o0 + j));
      }
      f32x4 y[NO];
      gemm_om_blocks<N1, NO, PR>(y, uf, lds + P::M2, lane, o0);
      if (ok) {
#pragma unroll
        for (int j = 0; j < NO; ++j) {
          const int c = g4 + 16 * (o0 + j);
          f32x4 v = y[j];
          if constexpr (MODE == ATOM_UPDATE_FWD) v += res[j] + v4(V2, c);
          *reinterpret_cast<f32x4*>(g.Y + (size_t)atom * D + c) = v;
        }
      }
    }
    {
      const int tn = t + (int)gridDim.x * 4;
      if (tn < ntiles) fetch(tn, in);
    }
    __syncthreads();
  }
}

template <int D, int N1, int PR>
struct AtomKernels {
  static constexpr int kD = D, kN1 = N1, kPR = PR;
  using P = AtomPlan<D, N1, PR>;
  // the four-wave split: fp32 operands, both layers in 64-wide multiples
  static constexpr bool kSplit = PR == PREC_F32 && N1 % 64 == 0 && D % 64 == 0;
  template <int MODE>
  static hipError_t allow() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_atom<D, N1, MODE, PR>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, P::IMG);
    if constexpr (kSplit) {
      if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_atom_split<D, N1, MODE, PR>),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                AtomSplitPlan<D, N1, MODE, PR>::TOTAL);
    }
    return e;
  }
  // the update networks exist for N1 == D; the readout for N1 = H in
  // {32, 64}, H == D = 64 included
  static constexpr bool kReadout = N1 <= 64;
  static hipError_t prepare() {
    hipError_t e = hipSuccess;
    if constexpr (kReadout) e = allow<ATOM_READOUT>();
    if constexpr (D == N1) {
      if (e == hipSuccess) e = allow<ATOM_UPDATE_FWD>();
      if (e == hipSuccess) e = allow<ATOM_UPDATE_BWD>();
    }
    return e;
  }
  template <int MODE>
  static void run(const AtomArgs& g, int G, int ntiles, int n_cu, hipStream_t s) {
    const dim3 grid(G), block(64 * kAtomNW);
    // at most two tiles per SIMD: the split kernel shortens the longest SIMD's work
    if constexpr (kSplit) {
      if (ntiles <= 2 * 4 * n_cu) {
        constexpr int lds_bytes = AtomSplitPlan<D, N1, MODE, PR>::TOTAL;
        hipLaunchKernelGGL((k_atom_split<D, N1, MODE, PR>), grid, block, lds_bytes, s, g);
        return;
      }
    }
    hipLaunchKernelGGL((k_atom<D, N1, MODE, PR>), grid, block, P::IMG, s, g);
  }
  static hipError_t launch(const AtomArgs& g, int n_cu, hipStream_t s) {
    const int ntiles = (g.M + kAtoms - 1) / kAtoms;
    int G = ntiles;
    if (G > n_cu) G = n_cu;
    if (G < 1) G = 1;
    if (g.mode == ATOM_READOUT) {
      if constexpr (kReadout) run<ATOM_READOUT>(g, G, ntiles, n_cu, s);
      else return hipErrorInvalidValue;
    } else if constexpr (D == N1) {   // the update networks
      if (g.mode == ATOM_UPDATE_FWD) run<ATOM_UPDATE_FWD>(g, G, ntiles, n_cu, s);
      else if (g.mode == ATOM_UPDATE_BWD) run<ATOM_UPDATE_BWD>(g, G, ntiles, n_cu, s);
      else return hipErrorInvalidValue;
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
};

// Atom-wise operands: fp16 when every MLP is 16-bit (PREC_F16S); fp16 pairs,
// which give fp32-grade products, when the model's products run on pairs
// (PREC_F16X2) and also behind a bfloat16 filter (PREC_BF16), whose
// atom-wise layers stay fp32-grade; fp32 otherwise.
template <class R, class F>
static R atom_dispatch(int D, int N1, int prec, R fail, F f) {
#define SN_AT(DD, NN, PP) \
  if (D == DD && N1 == NN && ap == PP) return f(AtomKernels<DD, NN, PP>{});
#define SN_AT_P(PP) \
  SN_AT(64, 64, PP) SN_AT(128, 128, PP) SN_AT(64, 32, PP) SN_AT(128, 32, PP) SN_AT(128, 64, PP)
  const int ap = prec == PREC_F16S                          ? PREC_F16S
                 : (prec == PREC_F16X2 || prec == PREC_BF16) ? PREC_F16X2
                                                             : PREC_F32;
  SN_AT_P(PREC_F32) SN_AT_P(PREC_F16S) SN_AT_P(PREC_F16X2)
#undef SN_AT_P
#undef SN_AT
  return fail;
}

hipError_t atom_prepare(int D, int H, int prec) {
  hipError_t e = atom_dispatch(D, D, prec, hipErrorInvalidValue,
                               [](auto k) { return decltype(k)::prepare(); });
  if (e != hipSuccess) return e;
  return atom_dispatch(D, H, prec, hipErrorInvalidValue,
                       [](auto k) { return decltype(k)::prepare(); });
}
size_t atom_image_bytes(int D, int N1, int prec) {
  return atom_dispatch(D, N1, prec, (size_t)0,
                       [](auto k) { return (size_t)decltype(k)::P::IMG; });
}
void atom_fill_image(int mode, int D, int N1, int prec, const float* W1, const float* b1,
                     const float* W2, const float* b2, unsigned char* out) {
  atom_dispatch(D, N1, prec, 0, [&](auto k) {
    using K = decltype(k);
    fill_atom_image<K::kD, K::kN1, K::kPR>(mode, W1, b1, W2, b2, out);
    return 0;
  });
}
hipError_t launch_atom(const AtomArgs& g, int D, int N1, int prec, int n_cu, hipStream_t s) {
  return atom_dispatch(D, N1, prec, hipErrorInvalidValue,
                       [&](auto k) { return decltype(k)::launch(g, n_cu, s); });
}

// E_r = sum over the replica's atoms of eps_i, accumulated in double in a
// fixed order: thread t keeps four partial sums over the atoms t + 1024 q
// (q mod 4 selecting the sum), then a fixed tree over the block.
constexpr int kEnergyThreads = 1024;

// Blocks 0 .. n_rep - 1: one replica's energy each (a double sum of its
// per-atom energies); the blocks after them: F = -(sum over the T blocks of
// dE/dr), kEnergyThreads components per block, and, when vel is given, the
// closing velocity half-kick of a BAOAB step, vel += half_kick F.
__global__ __launch_bounds__(kEnergyThreads) void k_finish(const float* eps, int n_rep, int n_per,
                                                           float* energy, const float* fb, int T,
                                                           int64_t n3, float* forces, float* vel,
                                                           float half_kick, const int32_t* rowptr,
                                                           int G0, int G, const float* side_f,
                                                           int64_t side_stride, DevStatus* st) {
  if ((int)blockIdx.x >= n_rep) {
    const int64_t k = (int64_t)(blockIdx.x - n_rep) * kEnergyThreads + threadIdx.x;
    if (k >= n3) return;
    const int64_t i = k / 3;
    const int c = (int)(k - 3 * i);
    int w0 = 0, w1 = 0, v0 = 0, v1 = 0;   // cut parts of blocks t > 0 and of block 0
    if (side_f) {
      const int64_t E = rowptr[n3 / 3];
      cut_workers(rowptr[i], rowptr[i + 1], (E + 15) / 16, G, w0, w1);
      cut_workers(rowptr[i], rowptr[i + 1], (E + 15) / 16, G0, v0, v1);
    }
    float s = 0.f;
    for (int t = 0; t < T; ++t) {
      float v = fb[(int64_t)t * n3 + k];
      const int a = t == 0 ? v0 : w0, b = t == 0 ? v1 : w1;
      if (a < b) {   // block t's row completed by the other workers' parts
        float acc = 0.f;
        for (int w = a; w < b; ++w) acc += side_f[t * side_stride + 3 * w + c];
        v += acc;
      }
      s += v;
    }
    const float f = -s;
    forces[k] = f;
    if (vel) vel[k] += half_kick * f;
    return;
  }
  __shared__ double sm[kEnergyThreads];
  const int r = blockIdx.x;
  const float* e = eps + (int64_t)r * n_per;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  int i = threadIdx.x;
  for (; i + 3 * kEnergyThreads < n_per; i += 4 * kEnergyThreads) {
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += (double)e[i + q * kEnergyThreads];
  }
  for (int q = 0; i < n_per; i += kEnergyThreads, ++q) s[q] += (double)e[i];
  sm[threadIdx.x] = (s[0] + s[1]) + (s[2] + s[3]);
  __syncthreads();
  for (int w = kEnergyThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) sm[threadIdx.x] += sm[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float E = (float)sm[0];
    energy[r] = E;
    if (!isfinite(E)) dev_fail(st, SN_ERR_NONFINITE, r);
  }
}

hipError_t launch_finish(const float* eps, int n_rep, int n_per, float* energy, const float* fb,
                         int T, int64_t n_atoms, float* forces, float* vel, float half_kick,
                         const int32_t* rowptr, int G0, int G, const float* side_f,
                         int64_t side_stride, DevStatus* st, hipStream_t s) {
  const int64_t n3 = 3 * n_atoms;
  const int64_t nb = n_rep + (n3 + kEnergyThreads - 1) / kEnergyThreads;
  hipLaunchKernelGGL(k_finish, dim3((unsigned)nb), dim3(kEnergyThreads), 0, s, eps, n_rep, n_per,
                     energy, fb, T, n3, forces, vel, half_kick, rowptr, G0, G, side_f,
                     side_stride, st);
  return hipGetLastError();
}

} // namespace sn
