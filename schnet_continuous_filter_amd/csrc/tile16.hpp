// Building blocks of the 16x16 MFMA tile kernels: bounded buffer loads, the
// XOR-swizzled weight-image layouts, and products whose weights are the A
// operand read from LDS and whose activations are the B operand held in
// registers in the accumulator layout (lane = item + 16 g; lane group g holds
// rows 4g..4g+3 of every 16-row block).
#pragma once

#include "common.hpp"

namespace sn {

#define LN2F 0.69314718055994530942f
#define LOG2EF 1.44269504088896340736f

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// Bounded loads: an offset past the resource's size reads 0.
__device__ __forceinline__ float bload(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ int bload_i(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}
__device__ __forceinline__ f32x4 bload4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Wave-uniform read of a read-only int array through the scalar cache.
__device__ __forceinline__ int cload(const int32_t* p, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// A copy of v the compiler cannot see through. Addresses derived from it are
// recomputed where they are used instead of being hoisted out of the tile loop
// and held in registers for the whole kernel.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// v rounded to a float in a register: every later use starts from this one
// rounding, whatever the compiler contracts into those uses.
__device__ __forceinline__ float pinned(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ _Float16 pinned(_Float16 v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Copies BYTES (a multiple of 16) of a weight image from global memory into
// LDS with the NT threads of a work-group. Each thread issues up to sixteen
// 16-byte loads before it writes any of them, so the copy waits for one memory
// round trip per sixteen pieces, not one per piece. The caller synchronises the
// work-group before the image is read.
template <int BYTES, int NT>
__device__ __forceinline__ void stage_lds(const void* src, unsigned char* lds) {
  static_assert(BYTES % 16 == 0, "image is copied in 16-byte pieces");
  constexpr int N = BYTES / 16;
  constexpr int PER = (N + NT - 1) / NT;
  constexpr int B = 16;
  const f32x4* g = reinterpret_cast<const f32x4*>(src);
  f32x4* l = reinterpret_cast<f32x4*>(lds);
  const int t = (int)threadIdx.x;
#pragma unroll
  for (int j0 = 0; j0 < PER; j0 += B) {
    f32x4 v[B];
#pragma unroll
    for (int j = 0; j < B && j0 + j < PER; ++j) {
      const int i = t + (j0 + j) * NT;
      if ((j0 + j + 1) * NT <= N || i < N) v[j] = g[i];
    }
#pragma unroll
    for (int j = 0; j < B && j0 + j < PER; ++j) {
      const int i = t + (j0 + j) * NT;
      if ((j0 + j + 1) * NT <= N || i < N) l[i] = v[j];
    }
  }
}

// Receivers cut by worker boundaries. A CFConv launch with G workers over a
// list of E edges (T = ceil(E / 16) tiles) starts worker v at edge
// 16 floor(v T / G). Worker w holds a part of receiver r, whose edges are
// [a, b), when its end (worker w + 1's start) falls strictly inside (a, b);
// those workers form the range [w0, w1), empty when r is not cut.
__device__ __forceinline__ void cut_workers(int64_t a, int64_t b, int64_t T, int G, int& w0,
                                            int& w1) {
  w0 = 0;
  w1 = 0;
  if (b - a < 2) return;
  const int64_t j0 = a / 16 + 1, j1 = (b + 15) / 16;   // tile boundaries 16 j inside: j0 <= j < j1
  if (j0 >= j1) return;
  w0 = (int)((j0 * G + T - 1) / T) - 1;   // the first worker start past a, minus one
  w1 = (int)((j1 * G + T - 1) / T) - 1;   // the first worker start at or past b, minus one
}

// Orders this wave's LDS writes before its later LDS reads (wave-private data).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// e^x for x <= 0 and ln(y) for y in [1, 2], on the hardware exp2 / log2.
__device__ __forceinline__ float exp_neg(float x) { return __builtin_amdgcn_exp2f(x * LOG2EF); }
__device__ __forceinline__ float ln_1_2(float y) { return __builtin_amdgcn_logf(y) * LN2F; }

// Shifted softplus and its derivative (the logistic sigmoid) from
// t = exp(-|a|) and h = (1 + t) / 2 in (1/2, 1]:
//   ssp(a) = ln(1 + e^a) - ln 2 = max(a, 0) + ln 2 log2(h),
//   sigmoid(a) = 1 / (1 + e^-a) = (a >= 0 ? 1 : t) / (2 h).
// log2 of h near 1 needs no cancellation against ln 2.
__device__ __forceinline__ void ssp_sig(float a, float& s, float& sg) {
  const float t = exp_neg(-fabsf(a));
  const float h = fmaf(t, 0.5f, 0.5f);
  const float r = __builtin_amdgcn_rcpf(h);
  s = fmaf(LN2F, __builtin_amdgcn_logf(h), fmaxf(a, 0.f));
  sg = (a >= 0.f ? 0.5f : 0.5f * t) * r;
}
__device__ __forceinline__ float ssp(float a) {
  const float t = exp_neg(-fabsf(a));
  return fmaf(LN2F, __builtin_amdgcn_logf(fmaf(t, 0.5f, 0.5f)), fmaxf(a, 0.f));
}

// max(u, 0) for finite u as the median of (u, 0, FLT_MAX): one instruction
// on a product's output, which fmaxf would first canonicalise (+inf maps to
// FLT_MAX; a NaN u yields a NaN through the other terms of the softplus).
__device__ __forceinline__ float pos_part(float u) {
  return __builtin_amdgcn_fmed3f(u, 0.f, 3.40282347e38f);
}

// The same in base-2 units: for a pre-activation given as u = a log2 e,
//   ssp(a) / ln 2 = max(u, 0) + log2(h),  h = (1 + 2^-|u|) / 2,
//   sigmoid(a)    = (u >= 0 ? 1 : 2^-|u|) / (2 h),
// one multiply fewer per value than from a (the factors log2 e and ln 2
// are carried by the inputs and outputs of the products around it).
__device__ __forceinline__ void ssp2_sig(float u, float& s, float& sg) {
  const float t = __builtin_amdgcn_exp2f(-fabsf(u));
  const float h = fmaf(t, 0.5f, 0.5f);
  const float r = __builtin_amdgcn_rcpf(h);
  s = __builtin_amdgcn_logf(h) + pos_part(u);
  sg = (u >= 0.f ? 0.5f : 0.5f * t) * r;
}
__device__ __forceinline__ float ssp2(float u) {
  const float t = __builtin_amdgcn_exp2f(-fabsf(u));
  return __builtin_amdgcn_logf(fmaf(t, 0.5f, 0.5f)) + pos_part(u);
}

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Operand element type of each precision and its 8-wide vector.
template <int PR> struct PrecT { using E = float; };
template <> struct PrecT<PREC_BF16> { using E = __bf16; using V8 = bf16x8; };
template <> struct PrecT<PREC_F16S> { using E = _Float16; using V8 = f16x8; };
template <> struct PrecT<PREC_F16X2> { using E = _Float16; using V8 = f16x8; };

// XOR-swizzled offset of element (row, col) of a row-major array with RL
// elements per row: 16-byte chunks (4 fp32 or 8 bf16) trade places by row, so
// that the 16 rows one lane group reads at a common column hit distinct banks.
template <int RL>
__host__ __device__ __forceinline__ int sw4(int row, int col) {
  constexpr int M = (RL / 4 >= 16) ? 15 : RL / 4 - 1;
  return row * RL + ((((col >> 2) ^ (row & M)) << 2) | (col & 3));
}
template <int RL>
__host__ __device__ __forceinline__ int sw8(int row, int col) {
  constexpr int M = (RL / 8 >= 16) ? 15 : RL / 8 - 1;
  return row * RL + ((((col >> 3) ^ (row & M)) << 3) | (col & 7));
}
// bf16 chained products: position of contraction index k in its group of 32,
// so that lane group g finds the 8 k values its accumulator rows hold
// (4g..4g+3 of two consecutive 16-feature blocks) in one 16-byte run.
__host__ __device__ constexpr int perm32(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// B operands of a chained product from an accumulator-layout input: fp32 uses
// the accumulator registers directly; bf16 packs them once (k slot 8 g + t of
// step kk is register t % 4 of block 2 kk + t / 4).
template <int K, int PR>
struct Operand {   // 16-bit operands
  using V8 = typename PrecT<PR>::V8;
  using E = typename PrecT<PR>::E;
  V8 S[K / 32];
  __device__ __forceinline__ explicit Operand(const f32x4 (&s)[K / 16]) {
#pragma unroll
    for (int kk = 0; kk < K / 32; ++kk)
#pragma unroll
      for (int t = 0; t < 8; ++t) S[kk][t] = (E)s[2 * kk + (t >> 2)][t & 3];
  }
};
template <int K>
struct Operand<K, PREC_F32> {
  const f32x4 (&S)[K / 16];
  __device__ __forceinline__ explicit Operand(const f32x4 (&s)[K / 16]) : S(s) {}
};

// B operands of a chained product on fp16 pairs: each input value x is
// scaled by the power of two a, then written as hi + lo with hi = fp16(a x)
// and lo = fp16(a x - hi) (both rounded to nearest even; 22 significant bits
// in all while a x stays in fp16's normal range). a x is exact, so the two
// parts agree however the compiler forms them.
template <int K>
struct SplitOperand {
  f16x8 H[K / 32], L[K / 32];
  __device__ __forceinline__ SplitOperand(const f32x4 (&s)[K / 16], float a) {
#pragma unroll
    for (int kk = 0; kk < K / 32; ++kk)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float v = s[2 * kk + (t >> 2)][t & 3] * a;
        const _Float16 h = (_Float16)v;
        H[kk][t] = h;
        L[kk][t] = (_Float16)(v - (float)h);
      }
  }
};

// Per-lane element offsets of the A-operand reads of an output-major image
// with K elements per row. The swizzle XORs the 16-byte chunk index with the
// row's low 4 bits, so only the low 4 bits of the chunk vary per lane: four
// offsets (chunk group q) plus compile-time constants address every read.
// Build once per tile from the lane index.
template <int K, int PR>
struct ImgLanes {
  int off[4];
  __device__ __forceinline__ explicit ImgLanes(int lane) {
    const int grp = lane >> 4, e = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (PR != PREC_F32) off[q] = sw8<K>(e, 32 * q + 8 * grp);
      else off[q] = sw4<K>(e, 16 * q + 4 * grp);
    }
  }
};

// acc += sum_k M[16 nb + e][k] S[k] for one output block nb; M is an
// output-major image with K elements per row (fp32: sw4 rows; 16-bit: sw8
// rows with perm32 positions).
template <int K, int PR>
__device__ __forceinline__ void gemm_om_block(f32x4& acc, const Operand<K, PR>& op,
                                              const void* img, int nb,
                                              const ImgLanes<K, PR>& ln) {
  if constexpr (PR != PREC_F32) {
    static_assert(K / 32 <= 4, "chunk groups");
    using E = typename PrecT<PR>::E;
    using V8 = typename PrecT<PR>::V8;
    const E* M = reinterpret_cast<const E*>(img) + 16 * nb * K;
#pragma unroll
    for (int kk = 0; kk < K / 32; ++kk) {
      const V8 w = *reinterpret_cast<const V8*>(M + ln.off[kk]);
      acc = mfma16(w, op.S[kk], acc);
    }
  } else {
    const float* M = reinterpret_cast<const float*>(img) + 16 * nb * K;
#pragma unroll
    for (int kb = 0; kb < K / 16; ++kb) {
      // chunk 4 kb + g: bit 4 (kb >= 4) is untouched by the swizzle
      const f32x4 w = *reinterpret_cast<const f32x4*>(M + ln.off[kb & 3] + 64 * (kb >> 2));
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mfma16(w[r], op.S[kb][r], acc);
    }
  }
}

// acc = sum_k M[16 nb + e][k] S[k] with M = MH + ML and S = H + L given as
// fp16 pairs: the three products MH H + MH L + ML H (the ML L term is below
// the pairs' own rounding). MH and ML are 16-bit output-major images as in
// gemm_om_block. The fp16 products enter the fp32 accumulator without a
// correctly rounded sum: bits of a product far below the accumulator's
// magnitude are lost. So every small correction product (one lo factor) is
// summed first, while the accumulator is of its own size, and the hi*hi
// products last; those are exact 22-bit numbers on the final sum's grid.
template <int K>
__device__ __forceinline__ void gemm_split_block(f32x4& acc, const SplitOperand<K>& op,
                                                 const void* img_hi, const void* img_lo, int nb,
                                                 const ImgLanes<K, PREC_F16X2>& ln) {
  static_assert(K / 32 <= 4, "chunk groups");
  const _Float16* MH = reinterpret_cast<const _Float16*>(img_hi) + 16 * nb * K;
  const _Float16* ML = reinterpret_cast<const _Float16*>(img_lo) + 16 * nb * K;
  f16x8 wh[K / 32];
  acc = f32x4{};
#pragma unroll
  for (int kk = 0; kk < K / 32; ++kk) {
    wh[kk] = *reinterpret_cast<const f16x8*>(MH + ln.off[kk]);
    const f16x8 wl = *reinterpret_cast<const f16x8*>(ML + ln.off[kk]);
    acc = mfma16(wl, op.H[kk], acc);
    acc = mfma16(wh[kk], op.L[kk], acc);
  }
#pragma unroll
  for (int kk = 0; kk < K / 32; ++kk) acc = mfma16(wh[kk], op.H[kk], acc);
}

// All NOUT / 16 output blocks: out[nb] = sum_k M[16 nb + e][k] S[k] (k < K).
template <int K, int NOUT, int PR>
__device__ __forceinline__ void gemm_om(f32x4 (&out)[NOUT / 16], const f32x4 (&S)[K / 16],
                                        const void* img, const ImgLanes<K, PR>& ln) {
  const Operand<K, PR> op(S);
#pragma unroll
  for (int nb = 0; nb < NOUT / 16; ++nb) {
    f32x4 acc = f32x4{};
    gemm_om_block<K, PR>(acc, op, img, nb, ln);
    out[nb] = acc;
  }
}
// The same, with the lane offsets built from the lane index here.
template <int K, int NOUT, int PR>
__device__ __forceinline__ void gemm_om(f32x4 (&out)[NOUT / 16], const f32x4 (&S)[K / 16],
                                        const void* img, int lane_) {
  const ImgLanes<K, PR> ln(opaque(lane_));
  gemm_om<K, NOUT, PR>(out, S, img, ln);
}

// Host: output-major image of the K x N product matrix m(k, n) (zero for
// k >= Kin or n >= Nin) for precision PR, with the per-output-channel scales
// of PREC_F16S written to scale[N] (left alone otherwise). fp32: sw4 rows;
// bf16: rounded values at sw8 positions; f16: m / s_n rounded. PERM places
// 16-bit values at their perm32 positions (for chained-product operands).
// With scale == nullptr, PREC_F16S rounds m itself (the caller has divided
// by scales of its own).
template <int K, int PR, bool PERM = true, class F>
void om_image(int N, int Kin, int Nin, F m, unsigned char* out, float* scale) {
  for (int n = 0; n < N; ++n) {
    float s = 1.f;
    if constexpr (PR == PREC_F16S) {
      if (scale) {
        float amax = 0.f;
        for (int k = 0; k < Kin && n < Nin; ++k) amax = fmaxf(amax, fabsf(m(k, n)));
        s = pow2_scale(amax);
        scale[n] = s;
      }
    }
    for (int k = 0; k < K; ++k) {
      const float v = (k < Kin && n < Nin) ? m(k, n) : 0.f;
      if constexpr (PR == PREC_F32) {
        reinterpret_cast<float*>(out)[sw4<K>(n, k)] = v;
      } else if constexpr (PR == PREC_BF16) {
        reinterpret_cast<uint16_t*>(out)[sw8<K>(n, PERM ? perm32(k) : k)] = bf16_rne_bits(v);
      } else {
        reinterpret_cast<uint16_t*>(out)[sw8<K>(n, PERM ? perm32(k) : k)] = f16_rne_bits(v / s);
      }
    }
  }
}

} // namespace sn
