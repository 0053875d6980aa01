// Atom-wise layers: type embedding, update network with residual, readout,
// their gradients, and the per-replica energy sum.
//
// FlashSchNet §3.2 "SchNet model": atom types select the initial features;
// "CFConv message passing and aggregation": a point-wise update network with a
// residual connection follows every aggregation; "Energy readout": a per-atom
// network then a sum. §4.1 "Precision contract": energy accumulation in fp32
// or better (the replica sum here accumulates in double).
//
// The dense layers are [atoms x K] x [K x N] products on fp32 MFMA
// (v_mfma_f32_32x32x2_f32); each kernel chains the two layers of one network
// with its activation (or gate) in between.
#include "common.hpp"

namespace sn {

#define LN2F 0.69314718055994530942f

__device__ __forceinline__ float ssp_f(float a) {
  const float t = __expf(-fabsf(a));
  return fmaxf(a, 0.f) + __logf(1.f + t) - LN2F;
}
__device__ __forceinline__ float sigmoid_f(float a) {
  const float t = __expf(-fabsf(a));
  const float inv = __builtin_amdgcn_rcpf(1.f + t);
  return a >= 0.f ? inv : t * inv;
}

// ------------------------------------------------------------------ fused atom-wise pairs
// A work-group takes 32 atoms at a time. The A tile sits in LDS (fp32, K
// permuted per lane so one 16-byte load feeds four MFMAs); B operands come
// straight from the weight matrices in global memory (row-major [K][N], so a
// wave's 32 lanes read 128 contiguous bytes per row; the matrices stay in L2).
// Each kernel chains two products with the elementwise step between them in
// registers and the intermediate back in the same LDS tile.
constexpr int kRows = 32;

template <int K>
__device__ __forceinline__ f32x16 mma_lds_glb(const float* Ap, const float* __restrict__ W,
                                              int ldw, int c, int h) {
  f32x16 acc = f32x16{};
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 8) {
    const float* wp = W + (size_t)(k0 + 4 * h) * ldw + c;
    const float b0 = wp[0], b1 = wp[ldw], b2 = wp[2 * ldw], b3 = wp[3 * ldw];
    const f32x4 av = *reinterpret_cast<const f32x4*>(Ap + k0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, b0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, b1, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, b2, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, b3, acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ int blk_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// MODE: ATOM_UPDATE_FWD  a = h W1 + b1 (stored);  x' = x + ssp(a) W2 + b2
//       ATOM_UPDATE_BWD  g_a = (g_x W2^T) * sigmoid(a);  g_h = g_a W1^T   (W1, W2 given transposed)
//       ATOM_READOUT     o = x W1 + b1;  eps = ssp(o).w2 + b2;  g_x = (sigmoid(o) * w2) W1^T
template <int D, int N1, int MODE>
__global__ __launch_bounds__(kThreads) void k_atom(AtomArgs g) {
  constexpr int SA = D + 4;
  __shared__ __align__(16) float At[kRows * SA];
  __shared__ float Sh[MODE == ATOM_READOUT ? kRows * (N1 + 1) : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, li = lane & 31;
  const float* Ap = At + li * SA + 4 * h;
  for (int m0 = blockIdx.x * kRows; m0 < g.M; m0 += gridDim.x * kRows) {
    // A tile: rows m0.., D columns, float4 loads
    for (int idx = tid; idx < kRows * D / 4; idx += kThreads) {
      const int r = idx / (D / 4), k4 = idx - r * (D / 4);
      f32x4 v = f32x4{};
      if (m0 + r < g.M) {
        const size_t o = (size_t)(m0 + r) * D + 4 * k4;
        v = *reinterpret_cast<const f32x4*>(g.A + o);
        if constexpr (MODE == ATOM_UPDATE_BWD) {
          if (g.A2) v += *reinterpret_cast<const f32x4*>(g.A2 + o);
          if (g.Asum) *reinterpret_cast<f32x4*>(g.Asum + o) = v;
        }
      }
      *reinterpret_cast<f32x4*>(At + r * SA + 4 * k4) = v;
    }
    __syncthreads();
    f32x16 v1 = f32x16{};
    const int c1 = wave * 32 + li;
    if (wave < N1 / 32) {
      const f32x16 acc = mma_lds_glb<D>(Ap, g.W1, N1, c1, h);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + blk_row(r, h);
        const bool ok = m < g.M;
        const size_t o = (size_t)m * N1 + c1;
        if constexpr (MODE == ATOM_UPDATE_FWD) {
          const float a = acc[r] + g.b1[c1];
          if (ok) g.Aout[o] = a;
          v1[r] = ssp_f(a);
        } else if constexpr (MODE == ATOM_UPDATE_BWD) {
          v1[r] = ok ? acc[r] * sigmoid_f(g.S[o]) : 0.f;
        } else {
          const float z = acc[r] + g.b1[c1];
          const float w2 = g.w2[c1];
          Sh[blk_row(r, h) * (N1 + 1) + c1] = ssp_f(z) * w2;
          v1[r] = sigmoid_f(z) * w2;
        }
      }
    }
    __syncthreads();
    if (wave < N1 / 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) At[blk_row(r, h) * SA + c1] = v1[r];
    }
    __syncthreads();
    if constexpr (MODE == ATOM_READOUT) {
      const int r = tid >> 3, part = tid & 7;
      float s = 0.f;
      for (int k = part * (N1 / 8); k < (part + 1) * (N1 / 8); ++k) s += Sh[r * (N1 + 1) + k];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      if (part == 0 && m0 + r < g.M) g.eps[m0 + r] = s + g.b2s;
    }
    if (wave < D / 32) {
      const int c2 = wave * 32 + li;
      const f32x16 acc = mma_lds_glb<N1>(Ap, g.W2, D, c2, h);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + blk_row(r, h);
        if (m >= g.M) continue;
        const size_t o = (size_t)m * D + c2;
        if constexpr (MODE == ATOM_UPDATE_FWD) g.Y[o] = g.R[o] + acc[r] + g.b2[c2];
        else g.Y[o] = acc[r];
      }
    }
    __syncthreads();
  }
}

hipError_t launch_atom(const AtomArgs& g, int D, int N1, int n_cu, hipStream_t s) {
  const int tiles = (g.M + kRows - 1) / kRows;
  const int cap = 8 * n_cu;
  const dim3 grid(tiles < cap ? (tiles > 0 ? tiles : 1) : cap);
#define SN_ATOM(DD, NN, MM)                                                             \
  if (D == DD && N1 == NN && g.mode == MM) {                                            \
    hipLaunchKernelGGL((k_atom<DD, NN, MM>), grid, dim3(kThreads), 0, s, g);            \
    return hipGetLastError();                                                           \
  }
  SN_ATOM(64, 64, ATOM_UPDATE_FWD) SN_ATOM(64, 64, ATOM_UPDATE_BWD)
  SN_ATOM(128, 128, ATOM_UPDATE_FWD) SN_ATOM(128, 128, ATOM_UPDATE_BWD)
  SN_ATOM(64, 32, ATOM_READOUT) SN_ATOM(64, 64, ATOM_READOUT)
  SN_ATOM(128, 32, ATOM_READOUT) SN_ATOM(128, 64, ATOM_READOUT)
#undef SN_ATOM
  return hipErrorInvalidValue;
}

// x[i][:] = Emb[types[i]][:]
__global__ __launch_bounds__(kThreads) void k_embed(const int32_t* types, const float* emb, int n,
                                                    int D, int n_types, float* x, DevStatus* st) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)n * D) return;
  const int64_t i = idx / D;
  const int c = (int)(idx - i * D);
  int t = types[i];
  if (t < 0 || t >= n_types) {
    if (c == 0) dev_fail(st, SN_ERR_INVALID_ARG, i);
    t = 0;
  }
  x[idx] = emb[(int64_t)t * D + c];
}

hipError_t launch_embed(const int32_t* types, const float* emb, int n_atoms, int D, int n_types,
                        float* x, DevStatus* st, hipStream_t s) {
  const int64_t n = (int64_t)n_atoms * D;
  hipLaunchKernelGGL(k_embed, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                     types, emb, n_atoms, D, n_types, x, st);
  return hipGetLastError();
}

// E_r = sum over the replica's atoms of eps_i, accumulated in double in a fixed order.
__global__ __launch_bounds__(kThreads) void k_energy(const float* eps, int n_per, float* energy,
                                                     DevStatus* st) {
  __shared__ double sm[kThreads];
  const int r = blockIdx.x;
  double s = 0.0;
  for (int i = threadIdx.x; i < n_per; i += kThreads) s += (double)eps[(int64_t)r * n_per + i];
  sm[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) sm[threadIdx.x] += sm[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float E = (float)sm[0];
    energy[r] = E;
    if (!isfinite(E)) dev_fail(st, SN_ERR_NONFINITE, r);
  }
}

hipError_t launch_energy(const float* eps, int n_rep, int n_per, float* energy, DevStatus* st,
                         hipStream_t s) {
  hipLaunchKernelGGL(k_energy, dim3(n_rep), dim3(kThreads), 0, s, eps, n_per, energy, st);
  return hipGetLastError();
}

} // namespace sn
