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
// (v_mfma_f32_32x32x2_f32). A work-group stages the weight matrix in LDS once
// and loops over 64-atom tiles; each wave owns 32x32 output blocks and the
// elementwise prologue/epilogue of each mode is fused into the product.
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

size_t gemm_lds_bytes(int K, int N) {
  // weight region (max of plain [K][N+4] and transposed [N][K+4]) + A tile [64][K+4]
  const size_t w = (size_t)K * (N + 4) > (size_t)N * (K + 4) ? (size_t)K * (N + 4) : (size_t)N * (K + 4);
  const size_t a = (size_t)kTileAtoms * ((K > N ? K : N) + 4);
  return (w + a) * 4;
}

template <int K, int N, int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(GemmArgs g) {
  constexpr bool TR = (MODE == GEMM_T_SIGMOID || MODE == GEMM_T);
  constexpr int SWP = N + 4;           // plain weights [K][N+4]
  constexpr int SWT = K + 4;           // transposed weights [N][K+4]
  constexpr int SW = TR ? SWT : SWP;
  constexpr int SA = (K > N ? K : N) + 4;
  constexpr int NCB = N / 32, NBLK = 2 * NCB, NBW = (NBLK + 3) / 4;
  constexpr int WSZ = (K * SWP > N * SWT) ? K * SWP : N * SWT;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  float* Ws = reinterpret_cast<float*>(lds_raw);
  float* At = Ws + WSZ;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, li = lane & 31;
  if constexpr (TR) {
    for (int idx = tid; idx < N * K; idx += kThreads) {
      const int n = idx / K, k = idx - n * K;
      Ws[n * SWT + k] = g.W[idx];
    }
  } else {
    for (int idx = tid; idx < K * N; idx += kThreads) {
      const int k = idx / N, n = idx - k * N;
      Ws[k * SWP + n] = g.W[idx];
    }
  }
  __syncthreads();

  for (int m0 = blockIdx.x * kTileAtoms; m0 < g.M; m0 += gridDim.x * kTileAtoms) {
    for (int idx = tid; idx < kTileAtoms * K; idx += kThreads) {
      const int r = idx / K, k = idx - r * K;
      const int m = m0 + r;
      float v = m < g.M ? g.A[(size_t)m * K + k] : 0.f;
      if constexpr (MODE == GEMM_SSP_RESID) v = ssp_f(v);
      At[r * SA + k] = v;
    }
    __syncthreads();
    f32x16 accs[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      const int blk = wave + 4 * q;
      accs[q] = f32x16{};
      if (blk >= NBLK) continue;
      const int rb = blk / NCB, cb = blk % NCB;
      const int c = cb * 32 + li;
      f32x16 acc = f32x16{};
      const float* ap = At + (rb * 32 + li) * SA + 4 * h;
      for (int k0 = 0; k0 < K; k0 += 8) {
        float b0, b1, b2, b3;
        if constexpr (TR) {
          const f32x4 bv = *reinterpret_cast<const f32x4*>(Ws + c * SWT + k0 + 4 * h);
          b0 = bv.x; b1 = bv.y; b2 = bv.z; b3 = bv.w;
        } else {
          const float* wp = Ws + (k0 + 4 * h) * SWP + c;
          b0 = wp[0]; b1 = wp[SWP]; b2 = wp[2 * SWP]; b3 = wp[3 * SWP];
        }
        const f32x4 av = *reinterpret_cast<const f32x4*>(ap + k0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, b0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, b1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, b2, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, b3, acc, 0, 0, 0);
      }
      const float bias = (MODE == GEMM_BIAS || MODE == GEMM_SSP_RESID || MODE == GEMM_READOUT)
                             ? g.bias[c] : 0.f;
      const float w2 = (MODE == GEMM_READOUT) ? g.w2[c] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int m = m0 + row;
        float y = acc[r];
        if constexpr (MODE == GEMM_READOUT) {
          const float z = y + bias;
          y = sigmoid_f(z) * w2;                 // d eps / d o
          accs[q][r] = ssp_f(z) * w2;            // this feature's share of eps
        }
        if (m >= g.M) continue;
        const size_t o = (size_t)m * N + c;
        if constexpr (MODE == GEMM_BIAS) y += bias;
        if constexpr (MODE == GEMM_SSP_RESID) y += bias + g.R[o];
        if constexpr (MODE == GEMM_T_SIGMOID) y *= sigmoid_f(g.S[o]);
        g.Y[o] = y;
      }
    }
    if constexpr (MODE == GEMM_READOUT) {
      // stage the shares after every wave finished reading the A tile
      __syncthreads();
#pragma unroll
      for (int q = 0; q < NBW; ++q) {
        const int blk = wave + 4 * q;
        if (blk >= NBLK) continue;
        const int rb = blk / NCB, c = (blk % NCB) * 32 + li;
#pragma unroll
        for (int r = 0; r < 16; ++r) At[(rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * SA + c] = accs[q][r];
      }
    }
    if constexpr (MODE == GEMM_READOUT) {
      __syncthreads();
      const int r = tid >> 2, part = tid & 3;
      float s = 0.f;
      for (int k = part * (N / 4); k < (part + 1) * (N / 4); ++k) s += At[r * SA + k];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      if (part == 0 && m0 + r < g.M) g.eps[m0 + r] = s + g.b2;
    }
    __syncthreads();
  }
}

template <int K, int N>
static void gemm_dispatch_mode(const GemmArgs& g, dim3 grid, size_t lds, hipStream_t s) {
  switch (g.mode) {
    case GEMM_BIAS: hipLaunchKernelGGL((k_gemm<K, N, GEMM_BIAS>), grid, dim3(kThreads), lds, s, g); break;
    case GEMM_SSP_RESID: hipLaunchKernelGGL((k_gemm<K, N, GEMM_SSP_RESID>), grid, dim3(kThreads), lds, s, g); break;
    case GEMM_T_SIGMOID: hipLaunchKernelGGL((k_gemm<K, N, GEMM_T_SIGMOID>), grid, dim3(kThreads), lds, s, g); break;
    case GEMM_T: hipLaunchKernelGGL((k_gemm<K, N, GEMM_T>), grid, dim3(kThreads), lds, s, g); break;
    case GEMM_READOUT: hipLaunchKernelGGL((k_gemm<K, N, GEMM_READOUT>), grid, dim3(kThreads), lds, s, g); break;
  }
}

template <int K, int N>
static hipError_t gemm_raise_limit() {
  const void* fns[] = {
      reinterpret_cast<const void*>(&k_gemm<K, N, GEMM_BIAS>),
      reinterpret_cast<const void*>(&k_gemm<K, N, GEMM_SSP_RESID>),
      reinterpret_cast<const void*>(&k_gemm<K, N, GEMM_T_SIGMOID>),
      reinterpret_cast<const void*>(&k_gemm<K, N, GEMM_T>),
      reinterpret_cast<const void*>(&k_gemm<K, N, GEMM_READOUT>)};
  for (const void* f : fns) {
    hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t gemm_prepare() {
  hipError_t e;
#define SN_RAISE(K, N) if ((e = gemm_raise_limit<K, N>()) != hipSuccess) return e;
  SN_RAISE(64, 64) SN_RAISE(128, 128) SN_RAISE(64, 32) SN_RAISE(128, 64) SN_RAISE(32, 64)
  SN_RAISE(64, 128) SN_RAISE(128, 32) SN_RAISE(32, 128)
#undef SN_RAISE
  return hipSuccess;
}

hipError_t launch_gemm(const GemmArgs& g, int n_cu, hipStream_t s) {
  const int tiles = (g.M + kTileAtoms - 1) / kTileAtoms;
  const int grid = tiles < n_cu ? (tiles > 0 ? tiles : 1) : n_cu;
  const size_t lds = gemm_lds_bytes(g.K, g.N);
  const dim3 gd(grid);
#define SN_CASE(KK, NN) if (g.K == KK && g.N == NN) { gemm_dispatch_mode<KK, NN>(g, gd, lds, s); return hipGetLastError(); }
  SN_CASE(64, 64) SN_CASE(128, 128) SN_CASE(64, 32) SN_CASE(128, 64) SN_CASE(32, 64)
  SN_CASE(64, 128) SN_CASE(128, 32) SN_CASE(32, 128)
#undef SN_CASE
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
