// HIP kernels for rollout-guided FP4 fake quantization on CDNA4 (gfx950).
//
// Paper: "TRACE: Rollout-Guided Quantization-Aware Training for FP4
// Reinforcement Learning of MoE Language Models" (arXiv 2610.07767).
//   §3.1 "Key Design" (Fig. 4(a)): block-scaled E2M1 rounding, the guided
//        selection between the two neighbouring codewords, its guarantee.
//   §3.2 "Key Design" (Fig. 6), §4.2: the compact mantissa-bit record.
//   Algorithm 1 prose: BracketFP4, Reconstruct, combined block/global scale.
//   §4.3: the MXFP4 (E8M0, 32-element block) variant.
//
// Every kernel streams its tensor once: one 16-byte load of 8 bf16 per lane
// ("unit"), consecutive lanes on consecutive units so each wave load is one
// contiguous 1 KiB run. An NVFP4 block (16 elements) is two lanes and an
// MXFP4 block (32) four; block maxima are exchanged with DPP quad
// permutations, with every lane of the wave executing them. No MFMA: the
// path is bound by HBM bandwidth, not by arithmetic.
//
// Arithmetic is binary32 with every operation rounded (built with
// -ffp-contract=off, denormals kept), so each step is exactly the one the
// header documents.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "trace_fp4_internal.h"

namespace tfp4 {
namespace {

constexpr int kUnroll = 4;              // units per thread per workgroup slab
constexpr float kFltMax = 3.40282346638528859812e+38f;

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ lane exchange

// Value of the partner lane (lane ^ 1) / (lane ^ 2) within each quad.
__device__ __forceinline__ uint32_t xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ uint32_t xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
}

// Largest bf16 magnitude (bits & 0x7FFF) among the 8 elements of a unit.
__device__ __forceinline__ uint32_t unit_amax_bits(const uint4& v) {
  us2 a = __builtin_bit_cast(us2, v.x & 0x7FFF7FFFu);
  us2 b = __builtin_bit_cast(us2, v.y & 0x7FFF7FFFu);
  us2 c = __builtin_bit_cast(us2, v.z & 0x7FFF7FFFu);
  us2 d = __builtin_bit_cast(us2, v.w & 0x7FFF7FFFu);
  us2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                    __builtin_elementwise_max(c, d));
  uint32_t mm = __builtin_bit_cast(uint32_t, m);
  return max(mm & 0xFFFFu, mm >> 16);
}

__device__ __forceinline__ uint32_t elem_bits(const uint4& v, int e) {
  uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// ------------------------------------------------------------ number formats

// bf16 magnitude bits -> binary32 value (exact).
__device__ __forceinline__ float mag_f32(uint32_t xb) { return __uint_as_float((xb & 0x7FFFu) << 16); }

// binary32 -> bf16 bits, round to nearest even (finite or +Inf input).
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  uint32_t b = __float_as_uint(v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// E2M1 magnitude of index k: 0, .5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_val(uint32_t k) {
  uint32_t b = (k + 252u) << 22;          // k >= 2: exponent/mantissa fields line up
  b = (k == 1u) ? 0x3F000000u : b;
  b = (k == 0u) ? 0u : b;
  return __uint_as_float(b);
}

// Round-to-nearest onto E2M1, ties to the even index, saturating at 6.
__device__ __forceinline__ uint32_t rtn_index(float t) {
  return (uint32_t)(t > 0.25f) + (uint32_t)(t >= 0.75f) + (uint32_t)(t > 1.25f) +
         (uint32_t)(t >= 1.75f) + (uint32_t)(t > 2.5f) + (uint32_t)(t >= 3.5f) +
         (uint32_t)(t > 5.0f);
}

// Largest k with v(k) <= t (7 for t >= 6): the lower end of BracketFP4.
__device__ __forceinline__ uint32_t floor_index(float t) {
  return (uint32_t)(t >= 0.5f) + (uint32_t)(t >= 1.0f) + (uint32_t)(t >= 1.5f) +
         (uint32_t)(t >= 2.0f) + (uint32_t)(t >= 3.0f) + (uint32_t)(t >= 4.0f) +
         (uint32_t)(t >= 6.0f);
}

// E4M3 (bias 7) byte of u in [0, 448], round to nearest even, subnormals kept.
__device__ __forceinline__ uint32_t e4m3_rne(float u) {
  uint32_t ub = __float_as_uint(u);
  // Normal range (u >= 2^-6): keep 3 mantissa bits, rebias the exponent 127 -> 7.
  uint32_t rn = ub + 0x7FFFFu + ((ub >> 20) & 1u);
  uint32_t nb = (rn >> 20) - (120u << 3);
  // Subnormal range: u * 2^9 rounded to an integer in [0, 8] (8 = 2^-6).
  float s = u * 512.0f + 8388608.0f;      // the add to 2^23 rounds to nearest even
  uint32_t sb = __float_as_uint(s) - 0x4B000000u;
  return (u < 0.015625f) ? sb : nb;
}

// E4M3 byte (sign ignored) -> value.
__device__ __forceinline__ float e4m3_value(uint32_t byte) {
  uint32_t ex = (byte >> 3) & 0xFu, m = byte & 7u;
  return ex == 0u ? (float)m * 0x1p-9f : ldexpf(1.0f + (float)m * 0.125f, (int)ex - 7);
}

// NVFP4 global scale from the tensor amax: 2688 / A, 1 for A == 0, <= FLT_MAX.
__device__ __forceinline__ float global_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  return fminf(2688.0f / amax, kFltMax);
}

// Per-workgroup table of the NVFP4 encode and decode factors of every E4M3
// scale byte under the call's S: lut[e] = {r = min(S/e, FLT_MAX), d = e/S},
// {0, 0} for e == 0. Replaces two divisions per block with one LDS read.
__device__ __forceinline__ void build_factor_lut(float2* lut, float S) {
  int i = threadIdx.x;
  if (i < 128) {
    float e = e4m3_value((uint32_t)i);
    float r = 0.0f, d = 0.0f;
    if (e != 0.0f) {
      d = e / S;
      r = fminf(S / e, kFltMax);
    }
    lut[i] = make_float2(r, d);
  }
}

// MXFP4 factors of an E8M0 byte: r = 2^-E, d = 2^E (exact).
__device__ __forceinline__ void mx_factors(uint32_t byte, float& r, float& d) {
  int E = (int)byte - 127;
  r = ldexpf(1.0f, -E);
  d = ldexpf(1.0f, E);
}

__device__ __forceinline__ uint32_t dequant_bits(uint32_t k, float d, uint32_t sign) {
  return bf16_rne(e2m1_val(k) * d) | (sign << 15);
}

// ------------------------------------------------------------ kernels

__global__ __launch_bounds__(64) void init_gscale_kernel(float* g) {
  if (threadIdx.x == 0) {
    g[0] = 1.0f;
    g[1] = 0.0f;
  }
}

// Tensor amax: max over bf16 magnitude bits; one atomic max per workgroup
// on the binary32 bits of A (monotonic for non-negative values).
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint4* __restrict__ x, int64_t units,
                                                        uint32_t* __restrict__ slot) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; u + 3 * stride < units; u += 4 * stride) {
    uint4 a = x[u], b = x[u + stride], c = x[u + 2 * stride], d = x[u + 3 * stride];
    m = max(m, max(max(unit_amax_bits(a), unit_amax_bits(b)),
                   max(unit_amax_bits(c), unit_amax_bits(d))));
  }
  for (; u < units; u += stride) m = max(m, unit_amax_bits(x[u]));
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = wmax[0];
    for (int w = 1; w < kThreads / 64; ++w) b = max(b, wmax[w]);
    atomicMax(slot, b << 16);
  }
}

// RTN quantization of one tensor (quantize_rtn / encode_guidance).
// FMT 0 NVFP4 / 1 MXFP4; PLANE 0 writes codes (u32 per unit), 1 writes the
// mantissa-bit plane (one byte per unit); WY writes y; SFA derives S from the
// amax in gsrc[1] and stores it to gsrc[0] (else S = gsrc[0]).
template <int FMT, int PLANE, bool WY, bool SFA>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint4* __restrict__ x, int64_t units,
                                                            float* gsrc, uint8_t* __restrict__ plane,
                                                            uint8_t* __restrict__ scales,
                                                            uint4* __restrict__ y) {
  __shared__ float2 lut[128];
  float S = 1.0f;
  if constexpr (FMT == 0) {
    if constexpr (SFA) {
      S = global_scale(gsrc[1]);
      if (blockIdx.x == 0 && threadIdx.x == 0) gsrc[0] = S;
    } else {
      S = gsrc[0];
    }
    build_factor_lut(lut, S);
    __syncthreads();
  }
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  uint4 v[kUnroll];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    int64_t u = base + j * kThreads;
    v[j] = u < units ? x[u] : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const int64_t u = base + j * kThreads;
    uint32_t bm = unit_amax_bits(v[j]);
    bm = max(bm, xor1(bm));
    if constexpr (FMT == 1) bm = max(bm, xor2(bm));
    float r, d;
    uint32_t sbyte;
    if constexpr (FMT == 0) {
      float a = __uint_as_float(bm << 16);
      float su = fminf((a / 6.0f) * S, 448.0f);
      sbyte = e4m3_rne(su);
      float2 rd = lut[sbyte & 0x7Fu];
      r = rd.x;
      d = rd.y;
    } else {
      int ef = (int)((bm >> 7) & 0xFFu);
      sbyte = (uint32_t)max(ef - 2, 0);
      mx_factors(sbyte, r, d);
    }
    uint32_t codes = 0, mbits = 0;
    uint32_t yw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t xb = elem_bits(v[j], e);
      uint32_t s = xb >> 15;
      float t = mag_f32(xb) * r;
      uint32_t k = rtn_index(t);
      codes |= ((s << 3) | k) << (4 * e);
      mbits |= (k & 1u) << e;
      if constexpr (WY) yw[e >> 1] |= dequant_bits(k, d, s) << (16 * (e & 1));
    }
    if (u < units) {
      if constexpr (PLANE == 0) reinterpret_cast<uint32_t*>(plane)[u] = codes;
      else plane[u] = (uint8_t)mbits;
      if constexpr (FMT == 0) {
        if ((u & 1) == 0) scales[u >> 1] = (uint8_t)sbyte;
      } else {
        if ((u & 3) == 0) scales[u >> 2] = (uint8_t)sbyte;
      }
      if constexpr (WY) y[u] = make_uint4(yw[0], yw[1], yw[2], yw[3]);
    }
  }
}

// Guided rounding under the rollout scales (guided_fake_quant) and the
// Reconstruct step alone (decode_guidance, DECODE = true).
// BITS 0: RTN; 1: compact (mantissa bit); 4: full rollout code.
template <int FMT, int BITS, bool DECODE, bool WCODES>
__global__ __launch_bounds__(kThreads) void guided_kernel(const uint4* __restrict__ x, int64_t units,
                                                          const uint8_t* __restrict__ guide,
                                                          const uint8_t* __restrict__ scales,
                                                          const float* __restrict__ gscale,
                                                          uint4* __restrict__ y,
                                                          uint32_t* __restrict__ codes_out) {
  __shared__ float2 lut[128];
  if constexpr (FMT == 0) {
    build_factor_lut(lut, gscale[0]);
    __syncthreads();
  }
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  uint4 v[kUnroll];
  uint32_t sb[kUnroll], g[kUnroll];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    int64_t u = base + j * kThreads;
    bool ok = u < units;
    v[j] = ok ? x[u] : make_uint4(0u, 0u, 0u, 0u);
    sb[j] = ok ? (uint32_t)scales[FMT == 0 ? (u >> 1) : (u >> 2)] : 0u;
    if constexpr (BITS == 1) g[j] = ok ? (uint32_t)guide[u] : 0u;
    else if constexpr (BITS == 4) g[j] = ok ? reinterpret_cast<const uint32_t*>(guide)[u] : 0u;
    else g[j] = 0u;
  }
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const int64_t u = base + j * kThreads;
    float r, d;
    if constexpr (FMT == 0) {
      float2 rd = lut[sb[j] & 0x7Fu];
      r = rd.x;
      d = rd.y;
    } else {
      mx_factors(sb[j], r, d);
    }
    uint32_t codes = 0;
    uint32_t yw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t xb = elem_bits(v[j], e);
      uint32_t s = xb >> 15;
      float t = mag_f32(xb) * r;
      uint32_t k;
      if constexpr (BITS == 0) {
        k = rtn_index(t);
      } else {
        uint32_t f = floor_index(t);
        bool inside = (t != e2m1_val(f)) && (f < 7u);
        if constexpr (BITS == 1) {
          uint32_t c = (g[j] >> e) & 1u;
          // The nearest magnitude of the other parity lies above t unless t is
          // in a dead zone, (2, 2.25) below 3 or (4, 4.5) below 6, where the
          // one below is nearer (ties go up).
          bool dead = (f == 4u && t < 2.25f) || (f == 6u && t < 4.5f);
          if constexpr (DECODE) {
            k = (c == (f & 1u)) ? f : ((f < 7u && !dead) ? f + 1u : f - 1u);
          } else {
            k = f + (uint32_t)(inside && c != (f & 1u) && !dead);
          }
        } else {
          uint32_t cr = (g[j] >> (4 * e)) & 0xFu;
          k = f + (uint32_t)(inside && (cr >> 3) == s && (cr & 7u) > f);
        }
      }
      codes |= ((s << 3) | k) << (4 * e);
      if constexpr (!DECODE) yw[e >> 1] |= dequant_bits(k, d, s) << (16 * (e & 1));
    }
    if (u < units) {
      if constexpr (DECODE || WCODES) codes_out[u] = codes;
      if constexpr (!DECODE) y[u] = make_uint4(yw[0], yw[1], yw[2], yw[3]);
    }
  }
}

// ------------------------------------------------------------ discrepancy sums

__device__ __forceinline__ double bf16_f64(uint32_t b) { return (double)__uint_as_float(b << 16); }

__device__ __forceinline__ void accum_unit(const uint4& a, const uint4& b, double& acc) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double d0 = bf16_f64(wa[i] & 0xFFFFu) - bf16_f64(wb[i] & 0xFFFFu);
    double d1 = bf16_f64(wa[i] >> 16) - bf16_f64(wb[i] >> 16);
    acc += d0 * d0;
    acc += d1 * d1;
  }
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Fixed-order sum of a workgroup's per-thread values; result valid in thread 0.
__device__ __forceinline__ void group_sum2(double& a, double& b) {
  __shared__ double sa[kThreads / 64], sbuf[kThreads / 64];
  a = wave_sum(a);
  b = wave_sum(b);
  if ((threadIdx.x & 63) == 0) {
    sa[threadIdx.x >> 6] = a;
    sbuf[threadIdx.x >> 6] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a = sa[0];
    b = sbuf[0];
    for (int w = 1; w < kThreads / 64; ++w) {
      a += sa[w];
      b += sbuf[w];
    }
  }
}

__global__ __launch_bounds__(kThreads) void stats_partial_kernel(const uint16_t* __restrict__ xt,
                                                                 const uint16_t* __restrict__ xr,
                                                                 const uint16_t* __restrict__ yt,
                                                                 const uint16_t* __restrict__ yr,
                                                                 int64_t n, double* __restrict__ partials) {
  const int64_t units = n / kUnitElems;
  const uint4* xt4 = reinterpret_cast<const uint4*>(xt);
  const uint4* xr4 = reinterpret_cast<const uint4*>(xr);
  const uint4* yt4 = reinterpret_cast<const uint4*>(yt);
  const uint4* yr4 = reinterpret_cast<const uint4*>(yr);
  double sb = 0.0, sf = 0.0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units; u += stride) {
    accum_unit(xt4[u], xr4[u], sb);
    accum_unit(yt4[u], yr4[u], sf);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int64_t i = units * kUnitElems; i < n; ++i) {
      double dx = bf16_f64(xt[i]) - bf16_f64(xr[i]);
      double dy = bf16_f64(yt[i]) - bf16_f64(yr[i]);
      sb += dx * dx;
      sf += dy * dy;
    }
  }
  group_sum2(sb, sf);
  if (threadIdx.x == 0) {
    partials[2 * blockIdx.x] = sb;
    partials[2 * blockIdx.x + 1] = sf;
  }
}

__global__ __launch_bounds__(kThreads) void stats_final_kernel(const double* __restrict__ partials,
                                                               int groups, int64_t n, double* acc3,
                                                               int accumulate) {
  double sb = 0.0, sf = 0.0;
  for (int i = threadIdx.x; i < groups; i += kThreads) {
    sb += partials[2 * i];
    sf += partials[2 * i + 1];
  }
  group_sum2(sb, sf);
  if (threadIdx.x == 0) {
    if (accumulate) {
      acc3[0] += sb;
      acc3[1] += sf;
      acc3[2] += (double)n;
    } else {
      acc3[0] = sb;
      acc3[1] = sf;
      acc3[2] = (double)n;
    }
  }
}

// ------------------------------------------------------------ launch plumbing

// Launch through hipLaunchKernel so the error code comes back to the caller
// instead of the thread's sticky "last error". Arguments are converted to the
// kernel's exact parameter types before their addresses are taken.
template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> typed(static_cast<P>(args)...);
  void* argv[sizeof...(P)];
  std::apply([&argv](auto&... e) {
    int i = 0;
    ((argv[i++] = static_cast<void*>(&e)), ...);
  }, typed);
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, s);
}

inline unsigned grid_for(int64_t units) {
  return (unsigned)((units + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll));
}

template <int FMT, int PLANE, bool WY, bool SFA>
hipError_t quant_dispatch(const uint16_t* x, int64_t units, float* gsrc, uint8_t* plane,
                          uint8_t* scales, uint16_t* y, hipStream_t s) {
  return launch(quantize_kernel<FMT, PLANE, WY, SFA>, dim3(grid_for(units)), dim3(kThreads), s,
                reinterpret_cast<const uint4*>(x), units, gsrc, plane, scales,
                reinterpret_cast<uint4*>(y));
}

template <int FMT, int PLANE>
hipError_t quant_dispatch_y(bool wy, bool sfa, const uint16_t* x, int64_t units, float* gsrc,
                            uint8_t* plane, uint8_t* scales, uint16_t* y, hipStream_t s) {
  if (wy) {
    return sfa ? quant_dispatch<FMT, PLANE, true, true>(x, units, gsrc, plane, scales, y, s)
               : quant_dispatch<FMT, PLANE, true, false>(x, units, gsrc, plane, scales, y, s);
  }
  return sfa ? quant_dispatch<FMT, PLANE, false, true>(x, units, gsrc, plane, scales, y, s)
             : quant_dispatch<FMT, PLANE, false, false>(x, units, gsrc, plane, scales, y, s);
}

template <int FMT, int BITS, bool DECODE, bool WCODES>
hipError_t guided_dispatch(const uint16_t* x, int64_t units, const uint8_t* guide,
                           const uint8_t* scales, const float* gscale, uint16_t* y, uint8_t* codes,
                           hipStream_t s) {
  return launch(guided_kernel<FMT, BITS, DECODE, WCODES>, dim3(grid_for(units)), dim3(kThreads), s,
                reinterpret_cast<const uint4*>(x), units, guide, scales, gscale,
                reinterpret_cast<uint4*>(y), reinterpret_cast<uint32_t*>(codes));
}

template <int FMT>
hipError_t guided_fmt(int bits, bool decode, const uint16_t* x, int64_t units, const uint8_t* guide,
                      const uint8_t* scales, const float* gscale, uint16_t* y, uint8_t* codes,
                      hipStream_t s) {
  if (decode) return guided_dispatch<FMT, 1, true, true>(x, units, guide, scales, gscale, y, codes, s);
  const bool wc = codes != nullptr;
  switch (bits) {
    case 0:
      return wc ? guided_dispatch<FMT, 0, false, true>(x, units, guide, scales, gscale, y, codes, s)
                : guided_dispatch<FMT, 0, false, false>(x, units, guide, scales, gscale, y, codes, s);
    case 1:
      return wc ? guided_dispatch<FMT, 1, false, true>(x, units, guide, scales, gscale, y, codes, s)
                : guided_dispatch<FMT, 1, false, false>(x, units, guide, scales, gscale, y, codes, s);
    default:
      return wc ? guided_dispatch<FMT, 4, false, true>(x, units, guide, scales, gscale, y, codes, s)
                : guided_dispatch<FMT, 4, false, false>(x, units, guide, scales, gscale, y, codes, s);
  }
}

}  // namespace

int64_t stats_groups(int64_t n) {
  int64_t units = n / kUnitElems;
  int64_t g = (units + (int64_t)kThreads * 4 - 1) / ((int64_t)kThreads * 4);
  if (g < 1) g = 1;
  if (g > kStatsMaxGroups) g = kStatsMaxGroups;
  return g;
}

hipError_t launch_global_scale(const uint16_t* x, int64_t units, float* gscale_out,
                               hipStream_t stream) {
  hipError_t e = launch(init_gscale_kernel, dim3(1), dim3(64), stream, gscale_out);
  if (e != hipSuccess || units == 0) return e;
  int64_t g = (units + (int64_t)kThreads * 8 - 1) / ((int64_t)kThreads * 8);
  if (g > 2048) g = 2048;
  return launch(amax_kernel, dim3((unsigned)g), dim3(kThreads), stream,
                reinterpret_cast<const uint4*>(x), units, reinterpret_cast<uint32_t*>(gscale_out + 1));
}

hipError_t launch_quantize(int fmt, int plane_mode, bool s_from_amax, const uint16_t* x,
                           int64_t units, float* gsrc, uint8_t* plane, uint8_t* scales,
                           uint16_t* y, hipStream_t stream) {
  if (units == 0) return hipSuccess;
  const bool wy = y != nullptr;
  if (fmt == 0) {
    return plane_mode == 0
               ? quant_dispatch_y<0, 0>(wy, s_from_amax, x, units, gsrc, plane, scales, y, stream)
               : quant_dispatch_y<0, 1>(wy, s_from_amax, x, units, gsrc, plane, scales, y, stream);
  }
  return plane_mode == 0
             ? quant_dispatch_y<1, 0>(wy, false, x, units, gsrc, plane, scales, y, stream)
             : quant_dispatch_y<1, 1>(wy, false, x, units, gsrc, plane, scales, y, stream);
}

hipError_t launch_guided(int fmt, int bits, bool decode_only, const uint16_t* x, int64_t units,
                         const uint8_t* guide, const uint8_t* scales, const float* gscale,
                         uint16_t* y, uint8_t* codes, hipStream_t stream) {
  if (units == 0) return hipSuccess;
  return fmt == 0 ? guided_fmt<0>(bits, decode_only, x, units, guide, scales, gscale, y, codes, stream)
                  : guided_fmt<1>(bits, decode_only, x, units, guide, scales, gscale, y, codes, stream);
}

hipError_t launch_stats(int64_t n, const uint16_t* xt, const uint16_t* xr, const uint16_t* yt,
                        const uint16_t* yr, double* acc3, int accumulate, double* partials,
                        hipStream_t stream) {
  const int groups = (int)stats_groups(n);
  hipError_t e = launch(stats_partial_kernel, dim3(groups), dim3(kThreads), stream, xt, xr, yt, yr,
                        n, partials);
  if (e != hipSuccess) return e;
  return launch(stats_final_kernel, dim3(1), dim3(kThreads), stream, (const double*)partials, groups,
                n, acc3, accumulate);
}

}  // namespace tfp4
