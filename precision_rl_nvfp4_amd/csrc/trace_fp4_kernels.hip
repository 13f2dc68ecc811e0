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
// Layout of the work. Each kernel streams its tensors: a lane owns "units"
// of 8 bf16 (one 16-byte load), consecutive lanes own consecutive units, so a
// wave load is one contiguous 1 KiB run. An NVFP4 block (16 elements) spans
// two lanes and an MXFP4 block (32) four; block maxima are exchanged with DPP
// quad permutations. A call may hold several global-scale groups: a
// workgroup tile lies inside one group (e.g. one 8192-token chunk of a
// streamed layer), holds several whole small groups (packed, e.g. one token's
// row), or is given by a table of row-offset groups (e.g. one expert's rows).
// Encoding with S derived from a group's amax reads the input once (packed
// groups, and chunk-sized groups in onepass_encode_kernel) or twice (larger
// groups). Data touched once is read and written with nontemporal accesses.
// No MFMA: the path is bound by HBM bandwidth.
//
// Per-element arithmetic. The budget at the HBM roofline is ~20 VALU
// operations per element, so the E2M1 work runs on gfx950's conversion
// instructions and on the 8 codes of a unit at once, as nibbles of a dword:
//   * t = x * r in binary32 (no FMA, denormals kept), exactly as specified;
//   * RTN(t)  = v_cvt_scalef32_pk_fp4_f32 with scale 1.0 (round to nearest
//     even index, saturating at 6, keeping the sign);
//   * floor(t) (the lower end of BracketFP4) = the stochastic-rounding
//     variant with zero random bits, which truncates the magnitude;
//   * t is a codeword  <=>  floor(t) != floor(pred(t)), pred(t) the next
//     binary32 value toward zero (a NaN pattern for t = +-0, which converts
//     to magnitude 7, so zero also reads as a codeword);
//   * bf16 results come from v_cvt_scalef32_pk_bf16_fp4 (exact decode; for
//     MXFP4 it applies the E8M0 scale exactly) and v_cvt_pk_bf16_f32 (RNE).
// These equivalences were checked against the CPU oracle on every boundary
// of the grid (and are re-checked bit for bit by the parity tests).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "trace_fp4_internal.h"

// Library-owned device memory: one copy per device, allocated when the code
// object is loaded there and held until the process ends. Host code reaches it
// only through the address hipGetSymbolAddress gives on each device (the names
// below stand for host-side shadows in host code).
//   g_wait_fails  count of the single-pass encode's bounded waits that gave up
//   scratch       the workspace of encode_guidance_noalloc (no caller memory)
static __device__ unsigned long long g_wait_fails;
static __device__ __align__(256) uint8_t scratch[tfp4::kScratchBytes];

namespace tfp4 {
namespace {

typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

constexpr float kFltMax = 3.40282346638528859812e+38f;
constexpr int kMidGroups = 64;          // first level of the partial-sum reduction
constexpr int64_t kDirectTiles = 65536; // up to this many per-tile pairs are summed in one level
// Tile of guided rounding and of the fused statistics (equal or packed
// groups): half the tile of the other kernels. Measured on a streamed
// layer: the fused pass 1-5% faster and plain guided rounding 1-5% faster
// than with kTileUnits, while Reconstruct alone, the encode with S supplied
// and a KV tensor's two-pass encode were 3-10% slower with the smaller tile,
// so those keep kTileUnits. The statistics with mismatch diagnostics keep
// the smaller tile too (2-5% slower than on kTileUnits), so that the sums
// are bit-identical with and without the diagnostics.
constexpr int64_t kGuidedTileUnits = kTileUnits / 2;
// Tile of a guided_kernel launch: kGuidedTileUnits for guided rounding and
// the fused statistics of equal or packed groups, kTileUnits otherwise.
constexpr int64_t guided_tile(bool decode, int map) { return (decode || map == 2) ? kTileUnits : kGuidedTileUnits; }
constexpr int kMismatchBins = 15;       // signed-grid distances 0..14
constexpr int kPackGroups = kTileUnits / 2;  // most groups in a packed tile (NVFP4: >= 2 units each)

// ------------------------------------------------------------ lane exchange

// Value of the partner lane (lane ^ 1) / (lane ^ 2) within each quad.
__device__ __forceinline__ uint32_t xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ uint32_t xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
}

// ------------------------------------------------------------ unit helpers

typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));

// Streaming accesses (data touched once): nontemporal, so they do not
// allocate in the caches.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const v4u_t v = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(uint4* p, const uint4& v) {
  const v4u_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<v4u_t*>(p));
}

// Largest bf16 magnitude (bits & 0x7FFF) among the 8 elements of a unit.
__device__ __forceinline__ uint32_t unit_amax_bits(const uint4& v) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  us2 a = __builtin_bit_cast(us2, v.x & 0x7FFF7FFFu);
  us2 b = __builtin_bit_cast(us2, v.y & 0x7FFF7FFFu);
  us2 c = __builtin_bit_cast(us2, v.z & 0x7FFF7FFFu);
  us2 d = __builtin_bit_cast(us2, v.w & 0x7FFF7FFFu);
  us2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  uint32_t mm = __builtin_bit_cast(uint32_t, m);
  return max(mm & 0xFFFFu, mm >> 16);
}

// The 8 bf16 of a unit as binary32 (exact). Element 2i is the low half of word i.
__device__ __forceinline__ void unit_f32(const uint4& v, float (&f)[8]) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

// ------------------------------------------------------------ E2M1 codes

// RTN codes of 8 signed values; element i in nibble i (bits 4i..4i+3).
__device__ __forceinline__ uint32_t rtn_codes(const float (&t)[8]) {
  uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, t[0], t[1], 1.0f, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, t[2], t[3], 1.0f, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, t[4], t[5], 1.0f, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, t[6], t[7], 1.0f, 3);
  return c;
}

// Codes of floor(|t|) onto the E2M1 magnitudes (sign kept). Only byte 0 of
// each conversion is defined, so the four bytes are gathered with v_perm.
__device__ __forceinline__ uint32_t floor_pair(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, (f2_t){a, b}, 0u, 1.0f, 0);
}
__device__ __forceinline__ uint32_t floor_codes(const float (&t)[8]) {
  const uint32_t s0 = floor_pair(t[0], t[1]), s1 = floor_pair(t[2], t[3]);
  const uint32_t s2 = floor_pair(t[4], t[5]), s3 = floor_pair(t[6], t[7]);
  const uint32_t lo = __builtin_amdgcn_perm(s1, s0, 0x0C0C0400u);  // [s0.b0, s1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(s3, s2, 0x0C0C0400u);  // [s2.b0, s3.b0, 0, 0]
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);               // [lo.b0, lo.b1, hi.b0, hi.b1]
}

// Mantissa bits (bit 0 of each nibble) of a code dword -> one byte, element i at bit i.
__device__ __forceinline__ uint32_t gather_mbits(uint32_t k) {
  uint32_t m = k & 0x11111111u;
  m = (m | (m >> 3)) & 0x03030303u;
  m = (m | (m >> 6)) & 0x000F000Fu;
  return (m | (m >> 12)) & 0xFFu;
}
// Inverse: bit i of a byte -> bit 0 of nibble i.
__device__ __forceinline__ uint32_t spread_bits(uint32_t c) {
  c = (c | (c << 12)) & 0x000F000Fu;
  c = (c | (c << 6)) & 0x03030303u;
  return (c | (c << 3)) & 0x11111111u;
}

// Low 2 bits of each nibble -> 16 bits, element i at bits 2i..2i+1.
__device__ __forceinline__ uint32_t gather_2bits(uint32_t k) {
  uint32_t m = k & 0x33333333u;
  m = (m | (m >> 2)) & 0x0F0F0F0Fu;
  m = (m | (m >> 4)) & 0x00FF00FFu;
  return (m | (m >> 8)) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t spread_2bits(uint32_t c) {
  c = (c | (c << 8)) & 0x00FF00FFu;
  c = (c | (c << 4)) & 0x0F0F0F0Fu;
  return (c | (c << 2)) & 0x33333333u;
}

// Low 3 bits of each nibble -> 24 bits, element i at bits 3i..3i+2.
__device__ __forceinline__ uint32_t gather_3bits(uint32_t k) {
  const uint32_t m = (k & 0x07070707u) | ((k & 0x70707070u) >> 1);  // 6 bits per byte
  return (m & 0x3Fu) | ((m >> 2) & 0xFC0u) | ((m >> 4) & 0x3F000u) | ((m >> 6) & 0xFC0000u);
}
__device__ __forceinline__ uint32_t spread_3bits(uint32_t c) {
  const uint32_t m = (c & 0x3Fu) | ((c & 0xFC0u) << 2) | ((c & 0x3F000u) << 4) | ((c & 0xFC0000u) << 6);
  return (m & 0x07070707u) | ((m & 0x38383838u) << 1);
}

// Training-side selection under the rollout scale for the 8 elements of a
// unit (t signed, carrying the training sign). Returns the chosen codes.
//   BITS 0: RTN.
//   BITS 1: compact record g = the rollout mantissa bits (byte). Of the
//           bracket {lo, hi} take hi when t lies strictly inside it, lo < 7,
//           hi's mantissa bit is the rollout's, and t is not in a dead zone
//           (2, 2.25) or (4, 4.5), where the Reconstruct reference is lo - 1.
//   BITS 2: g = the rollout's low 2 magnitude bits c (16 bits). The
//           reference is c + 4 when |t| reaches the midpoint of v(c) and
//           v(c + 4) (1, 1.75, 2.5, 3.75), else c; take hi when t is inside,
//           lo < 7 and the reference exceeds lo.
//   BITS 3: g = the rollout magnitudes (24 bits), the reference itself.
//   BITS 4: full record g = rollout codes (dword). Take hi when t is inside,
//           lo < 7, the signs agree and the rollout magnitude exceeds lo.
//   DECODE (BITS 1..3): the Reconstruct reference itself instead of the choice.
template <int BITS, bool DECODE>
__device__ __forceinline__ uint32_t select_codes(const float (&t)[8], uint32_t g) {
  if constexpr (BITS == 0) {
    return rtn_codes(t);
  } else if constexpr (BITS == 2 || BITS == 3) {
    const uint32_t L = floor_codes(t);
    uint32_t R;  // reference magnitudes, one per nibble
    if constexpr (BITS == 3) {
      R = spread_3bits(g);
    } else {
      R = spread_2bits(g);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t c = (R >> (4 * i)) & 3u;
        const uint32_t thr = 0x3F8u + ((0xFA60u >> (4 * c)) & 15u);  // midpoint bits >> 20
        R |= (uint32_t)(((__float_as_uint(t[i]) & 0x7FFFFFFFu) >> 20) >= thr) << (4 * i + 2);
      }
    }
    if constexpr (DECODE) return (L & 0x88888888u) | R;
    float tp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) tp[i] = __uint_as_float(__float_as_uint(t[i]) - 1u);
    const uint32_t Lp = floor_codes(tp);
    const uint32_t z = (L ^ Lp) & 0x77777777u;
    const uint32_t X = (z | (z >> 1) | (z >> 2)) & 0x11111111u;  // t is a codeword
    const uint32_t M = L & 0x77777777u;
    const uint32_t gt = ~((M | 0x88888888u) - R) & 0x88888888u;  // reference > lo
    // R > M is impossible when lo == 7, so no saturation mask is needed.
    return L + ((gt >> 3) & ~X);
  } else {
    const uint32_t L = floor_codes(t);
    float tp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) tp[i] = __uint_as_float(__float_as_uint(t[i]) - 1u);
    const uint32_t Lp = floor_codes(tp);
    const uint32_t z = (L ^ Lp) & 0x77777777u;
    const uint32_t X = (z | (z >> 1) | (z >> 2)) & 0x11111111u;  // t is a codeword
    const uint32_t M = L & 0x77777777u;
    const uint32_t S7 = M & (M >> 1) & (M >> 2) & 0x11111111u;   // lo == 7 (|t| >= 6)
    if constexpr (BITS == 4) {
      const uint32_t same_sign = ~(L ^ g) & 0x88888888u;
      const uint32_t r_gt = ~((M | 0x88888888u) - (g & 0x77777777u)) & 0x88888888u;
      return L + (((same_sign & r_gt) >> 3) & ~(X | S7));
    } else {
      const uint32_t P = (M ^ spread_bits(g)) & 0x11111111u;     // mantissa(lo) != c
      uint32_t D = 0;                                            // |t| in [2,2.25) or [4,4.5)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        D |= ((((__float_as_uint(t[i]) & 0x7F700000u) ^ 0x40000000u) - 1u) >> 31) << (4 * i);
      if constexpr (!DECODE) {
        return L + (P & ~(X | S7 | D));
      } else {
        // Reference = nearest magnitude with mantissa c, ties up: lo when c
        // matches; else hi, or lo - 1 in a dead zone or above 6; for a
        // codeword t the nearer neighbour, lo - 1 exactly for lo in {4, 6, 7}.
        const uint32_t Q = (M >> 2) & ((M >> 1) | ~M) & 0x11111111u;
        const uint32_t up = P & ((~X & ~(S7 | D)) | (X & ~Q));
        const uint32_t dn = P & ((~X & (S7 | D)) | (X & Q));
        return L + up - dn;
      }
    }
  }
}

// ------------------------------------------------------------ mismatch diagnostics

// Position of a code on the signed grid (-7..7; +-0 both 0).
__device__ __forceinline__ int code_pos(uint32_t c) {
  const int k = (int)(c & 7u);
  return (c & 8u) ? -k : k;
}

// Adds one unit's 8 elements to the workgroup histograms: distance between
// the guided and rollout codes (bins 1..14), between the RTN and rollout
// codes (bins 16..29), and the direction of guided vs RTN magnitudes (30, 31).
// Distance 0 is not counted here (it is the remainder of the tile).
// An element whose three codes agree adds to no bin, so only the elements
// where K or K0 differs from KR are visited (about 1% of them).
__device__ __forceinline__ void mismatch_unit(uint32_t K, uint32_t KR, uint32_t K0, uint32_t* hist) {
  uint32_t z = (K ^ KR) | (K0 ^ KR);
  z = (z | (z >> 1) | (z >> 2) | (z >> 3)) & 0x11111111u;   // bit 4i: element i differs
  while (z) {
    const int sh = __builtin_ctz(z);                          // 4i
    z &= z - 1u;
    const uint32_t kt = (K >> sh) & 15u, kr = (KR >> sh) & 15u, kb = (K0 >> sh) & 15u;
    const int pr = code_pos(kr);
    const int d1 = abs(code_pos(kt) - pr), d2 = abs(code_pos(kb) - pr);
    if (d1) atomicAdd(&hist[d1], 1u);
    if (d2) atomicAdd(&hist[kMismatchBins + d2], 1u);
    const uint32_t mt = kt & 7u, mb = kb & 7u;
    if (mt != mb) atomicAdd(&hist[mt > mb ? 2 * kMismatchBins : 2 * kMismatchBins + 1], 1u);
  }
}

// ------------------------------------------------------------ dequantization

template <int SEL>
__device__ __forceinline__ uint32_t dec_bf16(uint32_t codes, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, SEL));
}
template <int SEL>
__device__ __forceinline__ uint32_t dequant_nv_pair(uint32_t codes, float d) {
  const uint32_t v = dec_bf16<SEL>(codes, 1.0f);
  const f2_t p = {__uint_as_float(v << 16) * d, __uint_as_float(v & 0xFFFF0000u) * d};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf2_t));
}
// y = sign * bf16(v(k) * d) for the 8 codes (NVFP4: d any binary32).
__device__ __forceinline__ uint4 dequant_nv(uint32_t codes, float d) {
  return make_uint4(dequant_nv_pair<0>(codes, d), dequant_nv_pair<1>(codes, d),
                    dequant_nv_pair<2>(codes, d), dequant_nv_pair<3>(codes, d));
}
// MXFP4: d = 2^E applied exactly by the conversion (scale = E8M0 byte << 23).
__device__ __forceinline__ uint4 dequant_mx(uint32_t codes, float dscale) {
  return make_uint4(dec_bf16<0>(codes, dscale), dec_bf16<1>(codes, dscale),
                    dec_bf16<2>(codes, dscale), dec_bf16<3>(codes, dscale));
}

// ------------------------------------------------------------ scales

// NVFP4 global scale from the tensor amax: 2688 / A, 1 for A == 0, <= FLT_MAX.
__device__ __forceinline__ float global_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  return fminf(2688.0f / amax, kFltMax);
}

// E4M3 scale byte of a block with max magnitude bits `bm` (bf16):
// e = E4M3_RNE(min(fp32(fp32(a / 6) * S), 448)). fp32(a / 6) equals the
// binary64 product a * fl64(1/6) rounded once to binary32 for every bf16 a.
__device__ __forceinline__ uint32_t nv_scale_byte(uint32_t bm, float S) {
  const float a = __uint_as_float(bm << 16);
  const float q = (float)((double)a * (1.0 / 6.0));
  const float u = fminf(q * S, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(u, 0.0f, 0, false) & 0xFFu;
}

// E4M3 byte (0..127) -> value.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t ex = b >> 3, m = b & 7u;
  return ex == 0u ? (float)m * 0x1p-9f : __uint_as_float(((ex + 120u) << 23) | (m << 20));
}

// NVFP4 factors of one E4M3 byte under S: r = min(S / e, FLT_MAX), d = e / S,
// both 0 for e == 0 (the entries of build_factor_lut), for packed groups.
// Called by the two lanes of one block (adjacent lanes, even first, both
// active, with the same sb and S): each lane performs one of the two
// divisions and they swap results.
__device__ __forceinline__ void nv_factors_pair(uint32_t sb, float S, float& r, float& d) {
  const float e = e4m3_value(sb & 0x7Fu);
  const bool odd = (threadIdx.x & 1u) != 0u;
  const float num = odd ? e : S, den = odd ? S : e;
  float q = num / den;                 // even lane: S / e; odd lane: e / S
  if (!odd) q = fminf(q, kFltMax);
  if (e == 0.0f) q = 0.0f;
  const float o = __uint_as_float(xor1(__float_as_uint(q)));
  r = odd ? o : q;
  d = odd ? q : o;
}

// Workgroup table of the NVFP4 factors of every E4M3 byte under S:
// lut[e] = {r = min(S / e, FLT_MAX), d = e / S}, {0, 0} for e == 0.
__device__ __forceinline__ void build_factor_lut(float2* lut, float S) {
  const int i = threadIdx.x;
  if (i < 128) {
    const float e = e4m3_value((uint32_t)i);
    float r = 0.0f, d = 0.0f;
    if (e != 0.0f) {
      d = e / S;
      r = fminf(S / e, kFltMax);
    }
    lut[i] = make_float2(r, d);
  }
}

// MXFP4: E8M0 byte of a block with max magnitude bits bm:
// E = clamp(floor(log2 a) - 2, -127, 127), byte = E + 127.
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t bm) {
  return (uint32_t)max((int)((bm >> 7) & 0xFFu) - 2, 0);
}
// r = 2^-E (exact; 2^-127 is subnormal).
__device__ __forceinline__ float mx_r(uint32_t sb) {
  return __uint_as_float(sb >= 254u ? 0x00400000u : (254u - sb) << 23);
}
// Scale operand that makes the bf16 decode multiply by 2^E.
__device__ __forceinline__ float mx_dscale(uint32_t sb) { return __uint_as_float(sb << 23); }

// ------------------------------------------------------------ reductions

// Max over the wave's 64 lanes, returned to every lane; all lanes must be
// active. DPP within each row of 16 lanes (quad swaps, then rotations by 4
// and 8), then the four row maxima read as scalars: 4 DPP steps and 4 lane
// reads instead of 6 LDS permutes and their address arithmetic.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x124, 0xF, 0xF, false));  // row_ror:4
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x128, 0xF, 0xF, false));  // row_ror:8
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)m, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)m, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)m, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)m, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ double wave_sum(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Fixed-order sum of the workgroup's (NT threads) per-thread values; result
// valid in thread 0.
template <int NT = kThreads>
__device__ __forceinline__ void group_sum2(double& a, double& b) {
  __shared__ double sa[NT / 64], sbuf[NT / 64];
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
    for (int w = 1; w < NT / 64; ++w) {
      a += sa[w];
      b += sbuf[w];
    }
  }
}

// Sum of 8 non-negative binary32 terms, pairwise.
__device__ __forceinline__ float sum8(const float (&s)[8]) {
  return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

// sum_i (a_i - b_i)^2 over 8 pairs of binary32 values, returned as binary64.
// Fast path in binary32: each term passes through at most 5 roundings, so the
// relative error of the (non-negative) sum is below 5 * 2^-24. When the
// binary32 sum leaves [2^-100, FLT_MAX] (a square overflowed, or every term is
// tiny enough for underflow to matter) the unit is summed in binary64.
__device__ __forceinline__ double sq_diff_sum(const float (&a)[8], const float (&b)[8]) {
  float sq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float d = a[i] - b[i];
    sq[i] = d * d;
  }
  const float s = sum8(sq);
  if (s >= 0x1p-100f && s <= kFltMax) return (double)s;
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double d = (double)a[i] - (double)b[i];
    acc += d * d;
  }
  return acc;
}

// ------------------------------------------------------------ kernel arguments

// Work split of a launch. Normally a tile of tu units lies in one group
// (tiles = tiles per group). Packed (NVFP4 groups of a power-of-two unit
// count below tu, e.g. one token's row): a tile holds tu >> lg whole
// consecutive groups (tiles = tiles of the call).
// Row-offset groups (groups of any size, e.g. the experts of a grouped MoE
// input): a device table gives each workgroup its (group, tile); groups are
// the row ranges [offs[g], offs[g + 1]), tiles of group g are table entries
// tstart[g] .. tstart[g + 1] - 1, and entries past the last are (-1, 0).
struct TileMap {
  int64_t tu;         // units per tile
  int64_t upg;        // units per group
  int64_t tiles;      // tiles per group, or of the call when packed
  int64_t units;      // units of the call
  int64_t groups;     // groups of the call
  int lg;             // log2(upg) when packed
  int packed;
  // row-offset groups
  const int64_t* offs;   // [groups + 1] row offsets (clamped, nondecreasing)
  const int32_t* tstart; // [groups + 1] first table entry of each group
  const int2* table;     // [entries] (group, tile within the group)
  const uint32_t* tpart; // [entries] tile maxima (bf16 magnitude bits)
  int64_t upr;           // units per row
};

__device__ __forceinline__ void tile_of(const TileMap& m, int64_t& g, int64_t& tbase) {
  const int64_t b = blockIdx.x;
  g = b / m.tiles;
  tbase = (b - g * m.tiles) * m.tu;
}

struct AmaxArgs {
  const uint4* x;
  int64_t upg;
  int64_t g0;                // first group of this pass
  int nparts;                // workgroups (partials) per group
  uint32_t* part;            // [groups][kPartMax]
};

struct QuantArgs {
  TileMap map;
  int64_t g0;                // first group quantized by this launch
  int64_t qblocks;           // workgroups quantizing; the rest run `side`
  AmaxArgs side;             // amax pass of the next batch of groups
  const uint4* x;
  const float* gin;          // S of group g at gin[2g]
  float* gout;               // {S, A} per group
  const uint32_t* part;      // amax partials [groups][kPartMax]
  int nparts;                // partials per group
  uint8_t* plane;
  uint8_t* scales;
  uint4* y;
};

struct GuidedArgs {
  TileMap map;
  const uint4* x;
  const uint8_t* guide;
  const uint8_t* scales;
  const float* gscale;       // S of group g at gscale[2g]
  uint4* y;
  uint32_t* codes;
  const uint4* xr;           // rollout input (stats)
  double* partials;          // 2 per workgroup (stats)
  uint32_t* cpart;           // [kMismatchCounts][tiles] mismatch counts (diagnostics)
  uint32_t* ticket;          // counter of the split final sum, zeroed here (stats; or NULL)
};


// ------------------------------------------------------------ kernels

__global__ __launch_bounds__(64) void fill_gscale_kernel(float* g, int64_t groups) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (i < groups) {
    g[2 * i] = 1.0f;
    g[2 * i + 1] = 0.0f;
  }
}

// Partial group amax: workgroup w of group g writes the max bf16 magnitude
// (as binary32 bits) of its share of the group to part[g][w]. The share is a
// contiguous range of whole tiles of kThreads * 8 units, read a tile (32 KB
// per workgroup of NT threads) at a time. `blk` is the workgroup's index
// within the amax pass; `red` holds NT / 64 words.
template <int NT>
__device__ __forceinline__ void amax_body(const AmaxArgs& a, int64_t blk, uint32_t* red) {
  const int64_t gi = blk / a.nparts;
  const int w = (int)(blk - gi * a.nparts);
  const int64_t g = a.g0 + gi;
  const uint4* x = a.x + g * a.upg;
  constexpr int64_t kTile = (int64_t)kThreads * 8;
  const int64_t tiles = (a.upg + kTile - 1) / kTile;
  const int64_t per = (tiles + a.nparts - 1) / a.nparts;   // tiles of this workgroup
  const int64_t t0 = (int64_t)w * per;
  const int64_t t1 = min(t0 + per, tiles);
  uint32_t m = 0;
  for (int64_t t = t0; t < t1; ++t) {
    constexpr int U = (int)(kTile / NT);
    const int64_t base = t * kTile + threadIdx.x;
    uint4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t u = base + k * NT;
      v[k] = u < a.upg ? load_stream(x + u) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) m = max(m, unit_amax_bits(v[k]));
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int i = 1; i < NT / 64; ++i) r = max(r, red[i]);
    a.part[g * kPartMax + w] = r << 16;
  }
}

__global__ __launch_bounds__(kThreads) void amax_kernel(AmaxArgs a) {
  __shared__ uint32_t red[kThreads / 64];
  amax_body<kThreads>(a, blockIdx.x, red);
}

// Outputs of one quantized unit (global unit index gu): its guidance-plane
// bits, its block's scale byte (written by the block's first unit) and y.
template <int FMT, int PLANE, bool WY>
__device__ __forceinline__ void write_unit(uint32_t K, uint32_t sb, float d, float dsc, int64_t gu,
                                           uint8_t* plane, uint8_t* scales, uint4* y) {
  if constexpr (PLANE == 0) {
    // plane stored by the caller
  } else if constexpr (PLANE == 4) {
    __builtin_nontemporal_store(K, reinterpret_cast<uint32_t*>(plane) + gu);
  } else if constexpr (PLANE == 1) {
    __builtin_nontemporal_store((uint8_t)gather_mbits(K), plane + gu);
  } else if constexpr (PLANE == 2) {
    __builtin_nontemporal_store((uint16_t)gather_2bits(K), reinterpret_cast<uint16_t*>(plane) + gu);
  } else {
    const uint32_t w = gather_3bits(K);
    uint8_t* q = plane + 3 * gu;
    q[0] = (uint8_t)w;
    q[1] = (uint8_t)(w >> 8);
    q[2] = (uint8_t)(w >> 16);
  }
  if constexpr (FMT == 0) {
    if ((gu & 1) == 0) __builtin_nontemporal_store((uint8_t)sb, scales + (gu >> 1));
  } else {
    if ((gu & 3) == 0) __builtin_nontemporal_store((uint8_t)sb, scales + (gu >> 2));
  }
  if constexpr (WY) store_stream(y + gu, FMT == 0 ? dequant_nv(K, d) : dequant_mx(K, dsc));
}

// RTN quantization (quantize_rtn / encode_guidance).
// FMT 0 NVFP4 / 1 MXFP4; PLANE = bits of the guidance plane: 4 codes (u32 per
// unit), 1 mantissa bits (u8 per unit), 2 / 3 the low 2 / 3 magnitude bits
// (u16 / 3 bytes per unit); WY writes y; SSRC (NVFP4) 0: S = gin[2g]; 1: S from the amax
// partials, {S, A} stored to gout by the group's first tile. With SSRC 1 the
// workgroups past `qblocks` run the amax pass of the next batch of groups, so
// one launch quantizes batch b while reading batch b + 1 for its amax.
//
// PACK (NVFP4): the tile holds whole groups (see TileMap). SSRC 0: S of each
// group from gin; SSRC 2: from the group's own amax, reduced inside the
// workgroup, so the input is read once; {S, A} go to gout. The block factors
// are computed per block instead of from a table.
// Threads of a quantize_kernel workgroup; its tile is kTileUnits units either
// way. One group per tile (S supplied, from the amax partials or from the
// tile maxima of row-offset groups; MXFP4) runs 512 threads of 4 units (8
// waves per SIMD: 102.9 against 107.3 us for a streamed layer with S
// supplied); packed small groups keep 256 threads of 8 units (512 were
// slower there: 131 against 116 us).
constexpr int quant_threads(int ssrc, bool pack) { return (ssrc != 2 && !pack) ? 2 * kThreads : kThreads; }

template <int FMT, int PLANE, bool WY, int SSRC, bool PACK>
__global__ __launch_bounds__(quant_threads(SSRC, PACK)) void quantize_kernel(QuantArgs a) {
  constexpr int QT = quant_threads(SSRC, PACK), QU = (int)(kTileUnits / QT);
  __shared__ float2 lut[PACK ? 1 : 128];
  __shared__ uint32_t red[QT / 64];
  __shared__ float gs[PACK ? kPackGroups : 1];                  // S of the tile's groups
  __shared__ uint32_t ga[PACK && SSRC == 2 ? kPackGroups : 1];  // segment maxima (bf16 bits)
  if constexpr (SSRC == 1) {
    if ((int64_t)blockIdx.x >= a.qblocks) {
      amax_body<QT>(a.side, (int64_t)blockIdx.x - a.qblocks, red);
      return;
    }
  }
  int64_t g, tbase, gbase, lim;
  int tk = 0;  // tile within the group (row-offset groups)
  if constexpr (PACK) {
    g = 0;
    tbase = (int64_t)blockIdx.x * kTileUnits;
    gbase = 0;
    lim = a.map.units;
  } else if constexpr (SSRC == 3) {
    const int2 e = a.map.table[blockIdx.x];
    if (e.x < 0) return;
    g = e.x;
    tk = e.y;
    tbase = (int64_t)e.y * kTileUnits;
    gbase = a.map.offs[g] * a.map.upr;
    lim = a.map.offs[g + 1] * a.map.upr - gbase;
  } else {
    tile_of(a.map, g, tbase);
    g += a.g0;
    gbase = g * a.map.upg;
    lim = a.map.upg;
  }
  // Issue the tile's loads first; the scale and its factor table follow.
  uint4 v[QU];
#pragma unroll
  for (int j = 0; j < QU; ++j) {
    const int64_t u = tbase + j * QT + threadIdx.x;
    v[j] = u < lim ? load_stream(a.x + gbase + u) : make_uint4(0u, 0u, 0u, 0u);
  }
  float S = 1.0f;
  if constexpr (PACK) {
    const int lg = a.map.lg;
    const int64_t g0t = tbase >> lg;                 // first group of the tile
    const int gpt = kTileUnits >> lg;                // groups per tile
    if constexpr (SSRC == 2) {
      // Segments of min(upg, 64) lanes hold one group's units for a given j;
      // each writes its max to its own slot (tile unit >> lgs), so every slot
      // is written once and no atomics or clearing are needed. A group of
      // more than 64 units combines its 2^(lg - 6) slots.
      const int lgs = lg < 6 ? lg : 6;
      const int w = 1 << lgs;
#pragma unroll
      for (int j = 0; j < QU; ++j) {
        uint32_t bm = unit_amax_bits(v[j]);          // units past the end read as zero
        if (w == 64) {
          bm = wave_max_u32(bm);
        } else {
          for (int off = w >> 1; off > 0; off >>= 1) bm = max(bm, (uint32_t)__shfl_xor((int)bm, off));
        }
        if ((threadIdx.x & (w - 1)) == 0) ga[(j * QT + threadIdx.x) >> lgs] = bm;
      }
      __syncthreads();
      const int spg = 1 << (lg - lgs);               // slots per group
      for (int i = threadIdx.x; i < gpt; i += QT) {
        uint32_t gm = 0u;
        for (int k = 0; k < spg; ++k) gm = max(gm, ga[i * spg + k]);
        const float A = __uint_as_float(gm << 16);
        const float Sg = global_scale(A);
        gs[i] = Sg;
        const int64_t gg = g0t + i;
        if (gg < a.map.groups) {
          a.gout[2 * gg] = Sg;
          a.gout[2 * gg + 1] = A;
        }
      }
    } else {
      for (int i = threadIdx.x; i < gpt; i += QT) {
        const int64_t gg = g0t + i;
        gs[i] = gg < a.map.groups ? a.gin[2 * gg] : 1.0f;
      }
    }
    __syncthreads();
  } else if constexpr (FMT == 0) {
    if constexpr (SSRC == 3) {
      uint32_t m = 0;
      const int32_t t0 = a.map.tstart[g], t1 = a.map.tstart[g + 1];
      for (int i = t0 + (int)threadIdx.x; i < t1; i += QT) m = max(m, a.map.tpart[i]);
      m = wave_max_u32(m);
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
      __syncthreads();
      m = red[0];
      for (int i = 1; i < QT / 64; ++i) m = max(m, red[i]);
      const float A = __uint_as_float(m << 16);
      S = global_scale(A);
      if (tk == 0 && threadIdx.x == 0) {
        a.gout[2 * g] = S;
        a.gout[2 * g + 1] = A;
      }
    } else if constexpr (SSRC == 1) {
      uint32_t m = 0;
      for (int i = threadIdx.x; i < a.nparts; i += QT) m = max(m, a.part[g * kPartMax + i]);
      m = wave_max_u32(m);
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
      __syncthreads();
      m = red[0];
      for (int i = 1; i < QT / 64; ++i) m = max(m, red[i]);
      const float A = __uint_as_float(m);
      S = global_scale(A);
      if (tbase == 0 && threadIdx.x == 0) {
        a.gout[2 * g] = S;
        a.gout[2 * g + 1] = A;
      }
    } else {
      S = a.gin[2 * g];
    }
    build_factor_lut(lut, S);
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < QU; ++j) {
    const int64_t u = tbase + j * QT + threadIdx.x;
    uint32_t bm = unit_amax_bits(v[j]);
    bm = max(bm, xor1(bm));
    if constexpr (FMT == 1) bm = max(bm, xor2(bm));
    float r, d = 0.0f, dsc = 0.0f;
    uint32_t sb;
    if constexpr (PACK) {
      const float Sg = gs[(j * QT + threadIdx.x) >> a.map.lg];
      sb = nv_scale_byte(bm, Sg);
      nv_factors_pair(sb, Sg, r, d);
    } else if constexpr (FMT == 0) {
      sb = nv_scale_byte(bm, S);
      const float2 rd = lut[sb & 0x7Fu];
      r = rd.x;
      d = rd.y;
    } else {
      sb = mx_scale_byte(bm);
      r = mx_r(sb);
      dsc = mx_dscale(sb);
    }
    float f[8];
    unit_f32(v[j], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] *= r;
    const uint32_t K = rtn_codes(f);
    if constexpr (PLANE == 3) {
      // A wave whose 64 units are all in range and whose 192 plane bytes
      // start on a dword stores them as 48 dwords: dword l starts at bit
      // off = 32 l - 24 c of unit c = 4 l / 3 and ends in unit c + 1.
      const int64_t u0 = tbase + j * QT + (threadIdx.x & ~63);
      uint8_t* wp = a.plane + 3 * (gbase + u0);
      if (u0 + 64 <= lim && (reinterpret_cast<uintptr_t>(wp) & 3u) == 0) {
        const uint32_t w = gather_3bits(K);
        const int l = (int)threadIdx.x & 63;
        const int c = (4 * l) / 3;
        const int off = 32 * l - 24 * c;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * c, (int)w);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (c + 1), (int)w);
        if (l < 48) __builtin_nontemporal_store((lo >> off) | (hi << (24 - off)), reinterpret_cast<uint32_t*>(wp) + l);
        write_unit<FMT, 0, WY>(K, sb, d, dsc, gbase + u, a.plane, a.scales, a.y);
        continue;
      }
    }
    if (u < lim) write_unit<FMT, PLANE, WY>(K, sb, d, dsc, gbase + u, a.plane, a.scales, a.y);
  }
}

struct OnePassArgs {
  const uint4* x;
  int upg;                   // units per group (equal groups)
  int groups;
  int T;                     // equal groups: tiles (workgroups) per group; row-offset groups: tile workgroups W
  int Q;                     // equal groups: groups in flight
  int L;                     // units per tile (a multiple of 64, <= kOPTile); a group's last tile may be shorter
  int rounds;                // row-offset groups: rounds of every tile workgroup (even)
  int copies;                // published copies of each S (kSCopies for equal groups, 1 for row-offset groups)
  uint32_t* slots;           // tagged tile maxima: [groups][kPartMax] (equal groups) or [entries] (row-offset groups)
  uint32_t* sword;           // [groups][copies][64]: S bits at [.][c][0], 0 until published
  unsigned long long* fails; // bounded waits that gave up (device-wide count)
  int spin_max;              // polls before a wait gives up
  float* gout;
  uint8_t* plane;
  uint8_t* scales;
  uint4* y;
  // row-offset groups: the tile table built on the device from the offsets
  const int64_t* offs;       // [groups + 1] row offsets (clamped, nondecreasing)
  const int32_t* tstart;     // [groups + 1] first table entry of each group
  const int4* desc;          // [entries] tile descriptors {first unit (lo, hi), length, group}; group -1 past the last
  const int32_t* big;        // nonzero when a group has more tiles than stay on chip (see below)
  int entries;
  int upr;                   // units per row
};

constexpr int kSpinMax = 1 << 22;      // default bound of every wait, in polls (~0.25 s)
constexpr int kSCopies = 16;            // copies of each published S, one per 256-byte line
constexpr int kOPDataWaves = 11;                     // data waves per workgroup
constexpr int kOPData = kOPDataWaves * 64;           // data threads
constexpr int kOnePassThreads = kOPData + 64;        // + the control wave: 12 waves, 6 per SIMD with 2 per CU
constexpr int kOPUnits = 6;                          // units per data thread and tile
constexpr int kOPTile = kOPData * kOPUnits;          // most units per tile (4224, a multiple of 64)
constexpr int kOPTableTile = 4096;                   // tile of row-offset groups (a table entry)
// Every workgroup must become resident at once. Its waves are spread over a
// CU's 4 SIMDs, so a wave count that is not a multiple of 4 fills them
// unevenly, and a second workgroup per CU may not fit even where the
// occupancy query says it does (14 waves per workgroup: the launch stalls on
// its bounded waits).
static_assert((kOPDataWaves + 1) % 4 == 0, "single-pass workgroups must fill the 4 SIMDs of a CU evenly");
static_assert(kOPTableTile <= kOPTile && kOPTableTile % 64 == 0, "table tiles fit a single-pass tile");
constexpr int kSlotsPerLane = kPartMax / 64;
constexpr int kRawBufferWord3 = 0x00020000;     // buffer descriptor word 3: untyped 32-bit data, no swizzle
constexpr int kBufferNT = 2;                    // buffer access cache policy: nontemporal

__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Largest bf16 magnitude bits over units [u0, u1) of xg, read by one whole
// wave (all 64 lanes active, u0 and u1 the same in every lane) and returned
// to every lane: the slow path of a bounded wait that gave up. Four loads per
// lane are in flight at a time.
__device__ __forceinline__ uint32_t wave_units_amax(const uint4* xg, int64_t u0, int64_t u1) {
  const int64_t lane = threadIdx.x & 63;
  uint32_t m = 0;
  int64_t u = u0 + lane;
  for (; u + 3 * 64 < u1; u += 4 * 64) {
    const uint4 a = xg[u], b = xg[u + 64], c = xg[u + 128], d = xg[u + 192];
    m = max(max(m, unit_amax_bits(a)), max(unit_amax_bits(b), max(unit_amax_bits(c), unit_amax_bits(d))));
  }
  for (; u < u1; u += 64) m = max(m, unit_amax_bits(xg[u]));
  return wave_max_u32(m);
}

// The tile a workgroup handles in round r: its group (-1 for a padding
// round), its first unit in x, its length in units and its slot.
//   Equal groups: workgroup (q, t) takes tile t of groups q, q + Q, q + 2Q, ...
//   Row-offset groups: workgroup w takes table entries w, w + W, w + 2W, ...
//     (entries are the tiles of the groups in order, kOPTableTile units each).
struct OPTile {
  int g;
  int len;
  int64_t base;
  int64_t slot;
};

template <bool TABLE>
__device__ __forceinline__ OPTile op_tile(const OnePassArgs& a, int q, int t, int r) {
  OPTile d;
  if constexpr (TABLE) {
    const int e = t + r * a.T;
    d.g = -1;
    d.len = 0;
    d.base = 0;
    d.slot = e;
    if (e < a.entries) {
      const int4 td = a.desc[e];
      if (td.w >= 0) {
        d.g = td.w;
        d.base = (int64_t)(((uint64_t)(uint32_t)td.y << 32) | (uint32_t)td.x);
        d.len = td.z;
      }
    }
  } else {
    const int g = q + r * a.Q;
    const int t0u = t * a.L;
    const bool in = g < a.groups;
    d.g = in ? g : -1;
    d.len = in ? min(a.upg - t0u, a.L) : 0;
    d.base = (int64_t)(in ? g : 0) * a.upg + t0u;
    d.slot = (int64_t)g * kPartMax + t;
  }
  return d;
}

// The unit range [u0, u1) of group g in x.
template <bool TABLE>
__device__ __forceinline__ void op_group_range(const OnePassArgs& a, int g, int64_t& u0, int64_t& u1) {
  if constexpr (TABLE) {
    u0 = a.offs[g] * a.upr;
    u1 = a.offs[g + 1] * a.upr;
  } else {
    u0 = (int64_t)g * a.upg;
    u1 = u0 + a.upg;
  }
}

// First slot and number of slots (tiles) of group g.
template <bool TABLE>
__device__ __forceinline__ void op_group_slots(const OnePassArgs& a, int g, int64_t& s0, int64_t& ns) {
  if constexpr (TABLE) {
    s0 = a.tstart[g];
    ns = a.tstart[g + 1] - s0;
  } else {
    s0 = (int64_t)g * kPartMax;
    ns = a.T;
  }
}

// Unit range [u0, u1) of the tile behind slot `slot`, the i-th of group g.
template <bool TABLE>
__device__ __forceinline__ void op_slot_units(const OnePassArgs& a, int g, int64_t slot, int64_t i, int64_t& u0,
                                              int64_t& u1) {
  if constexpr (TABLE) {
    const int4 td = a.desc[slot];
    u0 = (int64_t)(((uint64_t)(uint32_t)td.y << 32) | (uint32_t)td.x);
    u1 = u0 + td.z;
  } else {
    u0 = (int64_t)g * a.upg + i * a.L;
    u1 = min(u0 + a.L, (int64_t)(g + 1) * a.upg);
  }
}

// Max over each row of 16 lanes, returned to every lane of the row; the
// row's lanes must be active.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x124, 0xF, 0xF, false));  // row_ror:4
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x128, 0xF, 0xF, false));  // row_ror:8
  return m;
}

// S and A of group g from its amax bits gm: {S, A} to gout and S to the
// group's published words (lane l < copies stores copy l).
template <bool TABLE>
__device__ __forceinline__ void publish_scale(const OnePassArgs& a, int g, uint32_t gm, int lane) {
  const float A = __uint_as_float(gm << 16);
  const float S = global_scale(A);
  if (lane < a.copies) store_agent(&a.sword[((int64_t)g * a.copies + lane) * 64], __float_as_uint(S));
  if (lane == 0) {
    a.gout[2 * (int64_t)g] = S;
    a.gout[2 * (int64_t)g + 1] = A;
  }
}

// Groups of at most this many tiles are combined by a 16-lane segment.
constexpr int kSegSlots = 128;

// A tile descriptor the control wave left in LDS, read into scalar registers
// (it is the same for every lane).
__device__ __forceinline__ OPTile uniform_tile(const OPTile& t) {
  OPTile d;
  d.g = __builtin_amdgcn_readfirstlane(t.g);
  d.len = __builtin_amdgcn_readfirstlane(t.len);
  const uint64_t b = (uint64_t)t.base, s = (uint64_t)t.slot;
  d.base = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b));
  d.slot = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(s >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)s));
  return d;
}

// Single-pass NVFP4 encode with S from each group's amax. The grid never
// exceeds the number of workgroups the device holds at once (2 per CU), so
// all of them are resident. Equal groups (TABLE false): Q sets of T
// workgroups (T tiles per group, sized at launch so every CU gets the same
// work) take groups q, q + Q, ... in turn, one tile per workgroup per group,
// kept on chip. Row-offset groups (TABLE true, e.g. one global scale per
// expert): W workgroups take the table's tiles w, w + W, ... in turn. One
// more workgroup combines.
//
// A tile workgroup is eleven data waves and one control wave (twelve waves:
// with two workgroups per CU every SIMD holds six, at most 85 VGPRs each).
// The data waves load, hold and quantize the tiles;
// the control wave does every wait on other workgroups. This split matters:
// a wait on memory is a wait on the wave's whole vector-memory counter,
// which also covers the tile loads in flight, so a data wave that polled
// would stall until its next tile had arrived.
//   * Data waves: a tile's max goes to its slot, tagged (bit 31), by one
//     store from the last of the eleven waves to reduce it (an LDS counter),
//     as soon as the tile has arrived; no barrier is involved.
//   * Combining workgroup (the last one): waits for each group's slots,
//     derives S and A, writes {S, A} to gout and publishes S (nonzero) to
//     `copies` words; its first wave takes the groups of more than
//     kSegSlots tiles in order, the other waves the smaller ones, 16 lanes
//     each. It runs ahead of the tiles, so S is combined as soon as the last
//     tile max of its group is in, about a round before it is needed.
//   * Control wave: waits for one S word of the round's group and builds the
//     table of block factors under S.
//   * One barrier per round: the data waves quantize a tile from its table
//     while the control wave prepares the next round's in the other half of
//     a double buffer.
// Three tiles are on chip per data wave: the one being quantized (in LDS,
// each thread keeping its own words), the next one (registers, max
// published) and the one after (registers, loads in flight). The two
// register tiles swap roles each round; within a round, unit j of the
// stashed tile is quantized, its LDS words refilled from the next tile and
// that register reloaded from the tile three rounds ahead, so the loads
// leave spread over the round rather than in one burst (a burst queues
// ahead of every other access of the CU, the slot stores and S polls
// included). Tiles are read through a buffer resource whose range is the
// tile, so every load instruction is issued whatever the tile's length and
// each wait covers exactly the older tile.
// A round's group is complete (all its slots published) once every
// workgroup has finished the round before, as long as a group spans at most
// one tile more than there are tile workgroups: always for equal groups
// (T <= W), and for row-offset groups whenever *big is 0. When a row-offset
// group is larger (the prep kernel sets *big; the routing may send most rows
// to one expert), every workgroup first reads all its tiles once to publish
// their maxima (one barrier per round), then runs the rounds above without
// publishing: the input is read twice, as in the two-pass schedule.
// Slots and S words are zeroed before the launch, by a fill kernel (equal
// groups) or by the kernel that builds the tile table. Every wait
// is bounded: past spin_max polls the waiting wave stops waiting, counts the
// give-up in *fails and takes what it waited for from the input itself (the
// maxima of the tiles whose slots were not tagged, or the whole group's
// amax), so the grid always drains and the results stay exact; only the
// time grows.
template <int PLANE, bool WY, bool TABLE>
__global__ __launch_bounds__(kOnePassThreads, 6) void onepass_encode_kernel(OnePassArgs a) {
  __shared__ float2 lut[2][128];
  __shared__ float sS[2];
  __shared__ OPTile ring[8];       // row-offset groups: the tile of round k at [k % 8], filled 4 rounds ahead
  __shared__ uint32_t wmax[2], wcnt[2];
  __shared__ uint4 stash[kOPUnits * kOPData];   // the tile being quantized (thread-private words)
  // Group and entry indices fit 31 bits (checked at launch), so the indexing
  // here is 32-bit where it can be, and mostly scalar.
  const int G = a.groups, Q = a.Q;
  const int W = TABLE ? a.T : a.Q * a.T;        // tile workgroups
  if ((int)blockIdx.x == W) {
    // ---- the combining workgroup (the last one): derives S of every group as
    // soon as the group's slots are tagged. Wave 0 takes the groups of more
    // than kSegSlots tiles, in order, all 64 lanes on one group; waves 1..11
    // take the smaller ones (e.g. the experts of a routed MoE layer) in
    // segments of 16 lanes, one group per segment, 44 groups at a time.
    const int cw = (int)threadIdx.x >> 6;
    if (cw == 0) {
      const int lane = (int)threadIdx.x;
      for (int g = 0; g < G; ++g) {
        int64_t s0, ns;   // first slot and number of slots of the group
        op_group_slots<TABLE>(a, g, s0, ns);
        if (ns <= kSegSlots) continue;   // empty (nobody waits for it), or a segment's
        uint32_t acc = 0;   // this lane's max over the group's slots (and over tiles read after a give-up)
        for (int64_t c0 = 0; c0 < ns; c0 += 64 * kSlotsPerLane) {
          uint32_t v[kSlotsPerLane];
#pragma unroll
          for (int k2 = 0; k2 < kSlotsPerLane; ++k2) {
            const int64_t i = c0 + lane + 64 * k2;
            v[k2] = i < ns ? load_agent(&a.slots[s0 + i]) : 0x80000000u;
          }
          int spins = 0;
          for (;;) {
            bool all = true;
#pragma unroll
            for (int k2 = 0; k2 < kSlotsPerLane; ++k2) all = all && (v[k2] & 0x80000000u) != 0u;
            if (__all(all)) break;
            if (++spins > a.spin_max) {
              // Some tiles' workgroups have not published (not resident beside
              // this one): take those tiles' maxima from x. An untagged slot
              // still holds 0 (cleared before the launch), so it adds nothing.
              if (lane == 0) atomicAdd(a.fails, 1ull);
#pragma unroll
              for (int k2 = 0; k2 < kSlotsPerLane; ++k2) {
                uint64_t miss = __ballot(c0 + lane + 64 * k2 < ns && (v[k2] & 0x80000000u) == 0u);
                while (miss != 0u) {
                  const int64_t i = c0 + __builtin_ctzll(miss) + 64 * k2;
                  miss &= miss - 1u;
                  int64_t u0, u1;
                  op_slot_units<TABLE>(a, g, s0 + i, i, u0, u1);
                  acc = max(acc, wave_units_amax(a.x, u0, u1));
                }
                v[k2] |= 0x80000000u;
              }
              break;
            }
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int k2 = 0; k2 < kSlotsPerLane; ++k2)
              if ((v[k2] & 0x80000000u) == 0u) v[k2] = load_agent(&a.slots[s0 + c0 + lane + 64 * k2]);
          }
#pragma unroll
          for (int k2 = 0; k2 < kSlotsPerLane; ++k2) acc = max(acc, v[k2] & 0x7FFFFFFFu);
        }
        publish_scale<TABLE>(a, g, wave_max_u32(acc), lane);
      }
      return;
    }
    // waves 1..11: one group of at most kSegSlots tiles per 16-lane segment
    const int seg = (cw - 1) * 4 + (((int)threadIdx.x & 63) >> 4);
    const int sl = (int)threadIdx.x & 15;
    const int segshift = (int)threadIdx.x & 48;   // the segment's first lane in the wave
    constexpr int kSegs = (kOnePassThreads / 64 - 1) * 4;
    for (int g = seg; g < G; g += kSegs) {
      int64_t s0, ns;
      op_group_slots<TABLE>(a, g, s0, ns);
      if (ns == 0 || ns > kSegSlots) continue;   // uniform in the segment
      uint32_t v[kSegSlots / 16];
#pragma unroll
      for (int k2 = 0; k2 < kSegSlots / 16; ++k2) {
        const int i = sl + 16 * k2;
        v[k2] = i < ns ? load_agent(&a.slots[s0 + i]) : 0x80000000u;
      }
      uint32_t late = 0;
      int spins = 0;
      for (;;) {
        bool all = true;
#pragma unroll
        for (int k2 = 0; k2 < kSegSlots / 16; ++k2) all = all && (v[k2] & 0x80000000u) != 0u;
        if (((__ballot(!all) >> segshift) & 0xFFFFu) == 0u) break;
        if (++spins > a.spin_max) {
          // as in wave 0: the untagged tiles' maxima from x, by the segment
          if (sl == 0) atomicAdd(a.fails, 1ull);
#pragma unroll
          for (int k2 = 0; k2 < kSegSlots / 16; ++k2) {
            uint32_t miss = (uint32_t)(__ballot(sl + 16 * k2 < ns && (v[k2] & 0x80000000u) == 0u) >> segshift) & 0xFFFFu;
            while (miss != 0u) {
              const int i = __builtin_ctz(miss) + 16 * k2;
              miss &= miss - 1u;
              int64_t u0, u1;
              op_slot_units<TABLE>(a, g, s0 + i, i, u0, u1);
              uint32_t m = 0;
              for (int64_t u = u0 + sl; u < u1; u += 16) m = max(m, unit_amax_bits(a.x[u]));
              late = max(late, row_max_u32(m));
            }
            v[k2] |= 0x80000000u;
          }
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int k2 = 0; k2 < kSegSlots / 16; ++k2)
          if ((v[k2] & 0x80000000u) == 0u) v[k2] = load_agent(&a.slots[s0 + sl + 16 * k2]);
      }
      uint32_t m = late;
#pragma unroll
      for (int k2 = 0; k2 < kSegSlots / 16; ++k2) m = max(m, v[k2] & 0x7FFFFFFFu);
      publish_scale<TABLE>(a, g, row_max_u32(m), sl);
    }
    return;
  }
  const int q = TABLE ? 0 : (int)blockIdx.x / a.T;
  const int t = TABLE ? (int)blockIdx.x : (int)blockIdx.x - q * a.T;
  // row-offset groups with a group larger than the grid holds: maxima first
  const bool maxima_first = TABLE && *a.big != 0;
  if (threadIdx.x == 0) {
    wmax[0] = wmax[1] = 0u;
    wcnt[0] = wcnt[1] = 0u;
  }
  __syncthreads();

  // Rounds this workgroup runs, padded to an even number (the data waves
  // run two rounds per iteration of a loop with one exit; a padding round
  // quantizes nothing).
  const int rounds = TABLE ? a.rounds : ((G - q + Q - 1) / Q + 1) & ~1;
  // wave index as a scalar, so the roles split without exec masking
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (wave == kOPDataWaves) {
    // ---- control wave
    const int lane = (int)threadIdx.x - kOPData;
    // Row-offset groups: the data waves take each round's tiles (the one
    // quantized, the one whose max is published, the one loaded) from a ring
    // in LDS, which this wave fills four rounds ahead, so the table loads
    // stay off their path. The ring slot a round writes is not read in the
    // round before or after it.
    if (TABLE && lane == 0)
      for (int k = 0; k < 4; ++k) ring[k] = op_tile<TABLE>(a, q, t, k);
    if (maxima_first)
      for (int k = 0; k < rounds; ++k) __syncthreads();   // the data waves' first read
    int par = 0;
    for (int k = 0; k < rounds; ++k, par ^= 1) {
      const OPTile d = TABLE ? uniform_tile(ring[k & 7]) : op_tile<TABLE>(a, q, t, k);
      // the tile of round k + 4 for the ring: its descriptor load is issued
      // now and written to LDS at the end of the round
      OPTile ahead{};
      if (TABLE && lane == 0) ahead = op_tile<TABLE>(a, q, t, k + 4);
      if (d.g < 0) {   // the data waves' padding round
        if (TABLE && lane == 0) ring[(k + 4) & 7] = ahead;
        __syncthreads();
        continue;
      }
      const int g = d.g;
      // S of group g, published by the combining workgroup (never 0)
      uint32_t v = 0u;
      if (lane == 0) {
        const uint32_t* w = &a.sword[((int64_t)g * a.copies + (int)(blockIdx.x % a.copies)) * 64];
        int spins = 0;
        while ((v = load_agent(w)) == 0u) {
          if (++spins > a.spin_max) {
            atomicAdd(a.fails, 1ull);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      v = (uint32_t)__shfl((int)v, 0);
      if (v == 0u) {
        // The wait gave up (the combining workgroup is not resident yet):
        // this wave reduces the whole group's amax from x itself; the same
        // exact maximum gives the same S the combining wave publishes.
        int64_t u0, u1;
        op_group_range<TABLE>(a, g, u0, u1);
        const uint32_t gm = wave_units_amax(a.x, u0, u1);
        v = __float_as_uint(global_scale(__uint_as_float(gm << 16)));
      }
      const float S = __uint_as_float(v);
      // factor table of every E4M3 byte under S: {min(S / e, FLT_MAX), e / S}
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = lane + 64 * h;
        const float e = e4m3_value((uint32_t)i);
        float r = 0.0f, dd = 0.0f;
        if (e != 0.0f) {
          dd = e / S;
          r = fminf(S / e, kFltMax);
        }
        lut[par][i] = make_float2(r, dd);
      }
      if (lane == 0) sS[par] = S;
      if (TABLE && lane == 0) ring[(k + 4) & 7] = ahead;
      __syncthreads();   // the round's table is ready; the one two rounds back is no longer read
    }
    return;
  }

  // ---- data waves
  // A round's tile is units base .. base + len - 1 of x; unit j of this
  // thread's share is base + tid + j * kOPData. Tiles are read through a
  // buffer resource whose range is the tile (empty in a padding round), so
  // units outside it read as zero without a memory access, and every tile
  // load is the same kOPUnits instructions.
  uint4 r0[kOPUnits], r1[kOPUnits];
  auto tile_rsrc = [&](const OPTile& d) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.x + (d.g >= 0 ? d.base : 0)), (short)0, d.len * 16,
                                             kRawBufferWord3);
  };
  auto load_tile = [&](uint4 (&v)[kOPUnits], const OPTile& d) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(d);
#pragma unroll
    for (int j = 0; j < kOPUnits; ++j)
      v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)threadIdx.x * 16,
                                                                              j * kOPData * 16, kBufferNT));
  };
  // Tile max of the round's tile -> its tagged slot, stored by the last data
  // wave to add its wave max (LDS counter `par`, reset by that wave).
  auto publish_max = [&](const uint4 (&v)[kOPUnits], const OPTile& d, int par) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kOPUnits; ++j) m = max(m, unit_amax_bits(v[j]));
    m = wave_max_u32(m);
    if (d.g >= 0 && (threadIdx.x & 63) == 0) {
      __hip_atomic_fetch_max(&wmax[par], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const uint32_t c = __hip_atomic_fetch_add(&wcnt[par], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (c == kOPDataWaves - 1) {
        const uint32_t M = __hip_atomic_load(&wmax[par], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        wmax[par] = 0u;
        wcnt[par] = 0u;
        store_agent(&a.slots[d.slot], 0x80000000u | M);
      }
    }
  };
  auto to_stash = [&](const uint4 (&v)[kOPUnits]) {
#pragma unroll
    for (int j = 0; j < kOPUnits; ++j) stash[j * kOPData + threadIdx.x] = v[j];
  };
  // Round k (publication counter `par` for round k + 2). On entry: stash =
  // tile of round k (max published), ra = tile of k + 1 (max published), rb
  // = loads of k + 2 in flight. On exit ra and rb have swapped roles. With
  // maxima_first every max is already published and none is published here.
  auto encode_round = [&](uint4 (&ra)[kOPUnits], uint4 (&rb)[kOPUnits], int k, int par) {
    __syncthreads();   // the control wave has the round's factor table (and row-offset tiles) ready
    // (equal groups: the tiles are plain arithmetic on the round index)
    const OPTile d = TABLE ? uniform_tile(ring[k & 7]) : op_tile<TABLE>(a, q, t, k);
    const bool live = d.g >= 0;
    const float S = sS[par];
    const float2* L = lut[par];
    // Outputs of this tile, through buffer resources whose range is the
    // tile: stores past it are dropped by the range check, and every
    // offset is 32-bit. The tile starts on an even unit, so a unit's parity
    // (which decides who writes the block's scale byte) is the lane's.
    constexpr int PB = PLANE == 4 ? 4 : PLANE == 3 ? 3 : PLANE == 2 ? 2 : 1;   // plane bytes per unit
    const int64_t gb = live ? d.base : 0;
    const int tl = live ? d.len : 0;
    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc(a.plane + gb * PB, (short)0, tl * PB, kRawBufferWord3);
    // 3-bit planes are stored a dword at a time where the tile's plane bytes
    // start on a dword; su and the wave offsets are multiples of 64 units.
    const bool al3 = PLANE == 3 && ((reinterpret_cast<uintptr_t>(a.plane + gb * PB) & 3u) == 0);
    const __amdgpu_buffer_rsrc_t rsc =
        __builtin_amdgcn_make_buffer_rsrc(a.scales + (gb >> 1), (short)0, tl >> 1, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t ryy =
        __builtin_amdgcn_make_buffer_rsrc(WY ? a.y + gb : a.y, (short)0, WY ? tl * 16 : 0, kRawBufferWord3);
    const int lane_u = (int)threadIdx.x;   // the thread's unit offset in the tile, for j = 0
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(TABLE ? uniform_tile(ring[(k + 3) & 7]) : op_tile<TABLE>(a, q, t, k + 3));
    // Unit by unit: quantize stash[j], refill it from ra[j] and reload ra[j]
    // from the tile of round k + 3, so the tile's loads leave over the whole
    // round rather than in one burst (a burst queues ahead of every other
    // access of the CU, the slot stores and S polls included).
#pragma unroll
    for (int j = 0; j < kOPUnits; ++j) {
      if (live) {
        const uint4 v = stash[j * kOPData + threadIdx.x];
        uint32_t bm = unit_amax_bits(v);
        bm = max(bm, xor1(bm));
        const uint32_t sb = nv_scale_byte(bm, S);
        const float2 rd = L[sb & 0x7Fu];
        float f[8];
        unit_f32(v, f);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] *= rd.x;
        const uint32_t K = rtn_codes(f);
        const int su = j * kOPData;   // the unit's offset in the tile, less the lane's
        if constexpr (PLANE == 4) {
          __builtin_amdgcn_raw_buffer_store_b32(K, rp, lane_u * 4, su * 4, kBufferNT);
        } else if constexpr (PLANE == 1) {
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)gather_mbits(K), rp, lane_u, su, kBufferNT);
        } else if constexpr (PLANE == 2) {
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)gather_2bits(K), rp, lane_u * 2, su * 2, kBufferNT);
        } else {
          const uint32_t w = gather_3bits(K);
          const int wu = lane_u & ~63;   // the wave's first unit, less su
          if (al3 && su + wu + 64 <= tl) {
            // The wave's 64 units are 192 contiguous, dword-aligned plane
            // bytes: lane l < 48 stores dword l, which starts at bit 32 l,
            // i.e. bit off = 32 l - 24 c of unit c = 4 l / 3, and takes the
            // rest of its 32 bits from unit c + 1.
            const int l = lane_u & 63;
            const int c = (4 * l) / 3;
            const int off = 32 * l - 24 * c;
            const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * c, (int)w);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (c + 1), (int)w);
            if (l < 48) __builtin_amdgcn_raw_buffer_store_b32((lo >> off) | (hi << (24 - off)), rp, wu * 3 + 4 * l, su * 3, kBufferNT);
          } else {
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)w, rp, lane_u * 3, su * 3, kBufferNT);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(w >> 8), rp, lane_u * 3 + 1, su * 3, kBufferNT);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(w >> 16), rp, lane_u * 3 + 2, su * 3, kBufferNT);
          }
        }
        if ((lane_u & 1) == 0) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, rsc, lane_u >> 1, su >> 1, kBufferNT);
        if constexpr (WY)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u_t, dequant_nv(K, rd.y)), ryy, lane_u * 16, su * 16,
                                                 kBufferNT);
      }
      stash[j * kOPData + threadIdx.x] = ra[j];
      ra[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)threadIdx.x * 16,
                                                                              j * kOPData * 16, kBufferNT));
      __builtin_amdgcn_sched_barrier(0);
    }
    // the tile after next: its loads were issued a round ago
    if (!maxima_first) publish_max(rb, TABLE ? uniform_tile(ring[(k + 2) & 7]) : op_tile<TABLE>(a, q, t, k + 2), par);
  };

  if (maxima_first) {
    // Every tile's max first: one tile at a time, one barrier per round (the
    // LDS counters of a round are reused two rounds later).
    for (int k = 0; k < rounds; ++k) {
      const OPTile d = op_tile<TABLE>(a, q, t, k);
      load_tile(r0, d);
      publish_max(r0, d, k & 1);
      __syncthreads();
    }
  }
  {
    const OPTile d0 = op_tile<TABLE>(a, q, t, 0), d1 = op_tile<TABLE>(a, q, t, 1), d2 = op_tile<TABLE>(a, q, t, 2);
    load_tile(r0, d0);
    if (!maxima_first) publish_max(r0, d0, 0);
    to_stash(r0);
    load_tile(r0, d1);
    load_tile(r1, d2);
    if (!maxima_first) publish_max(r0, d1, 1);
  }
  for (int k = 0; k < rounds; k += 2) {
    encode_round(r0, r1, k, 0);
    encode_round(r1, r0, k + 1, 1);
  }
}

__global__ __launch_bounds__(kThreads) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    p[i] = 0u;
}

// ---- row-offset groups (e.g. one global scale per expert of a grouped MoE input)

// Exclusive scan over the workgroup (max when MAXOP, else sum) of one value
// per thread, in thread order; *total gets the whole reduction. Identity 0
// (the values are >= 0).
template <bool MAXOP>
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* total) {
  __shared__ int64_t wtot[kThreads / 64];
  const int lane = (int)threadIdx.x & 63, w = (int)threadIdx.x >> 6;
  int64_t incl = v;
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t o = __shfl_up(incl, d);
    if (lane >= d) incl = MAXOP ? max(incl, o) : incl + o;
  }
  int64_t excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0;
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int64_t pre = 0, all = 0;
  for (int k = 0; k < kThreads / 64; ++k) {
    const int64_t t = wtot[k];
    if (k < w) pre = MAXOP ? max(pre, t) : pre + t;
    all = MAXOP ? max(all, t) : all + t;
  }
  *total = all;
  __syncthreads();   // wtot[] is reused by the next scan
  return MAXOP ? max(pre, excl) : pre + excl;
}

// One workgroup. From the caller's row offsets (read only here) it derives
// offs = the running max of clamp(off, 0, rows), so groups are disjoint row
// ranges, and tstart = the exclusive prefix sum of each group's tile count.
// Empty groups get {S, A} = {1, 0} in gout (if given): no tile writes them.
__global__ __launch_bounds__(kThreads) void offs_prep_kernel(const int64_t* __restrict__ off_in,
                                                            int64_t G, int64_t rows, int64_t upr,
                                                            int64_t* offs, int32_t* tstart, float* gout) {
  const int64_t n = G + 1;
  const int64_t per = (n + kThreads - 1) / kThreads;
  const int64_t i0 = min((int64_t)threadIdx.x * per, n), i1 = min(i0 + per, n);
  int64_t total;
  // 1. running max of the clamped offsets
  int64_t m = 0;
  for (int64_t i = i0; i < i1; ++i) m = max(m, min(max(off_in[i], (int64_t)0), rows));
  m = block_exclusive_scan<true>(m, &total);   // max over the entries before i0
  for (int64_t i = i0; i < i1; ++i) {
    m = max(m, min(max(off_in[i], (int64_t)0), rows));
    offs[i] = m;
  }
  __syncthreads();
  // 2. tiles per group, exclusive prefix sum
  const int64_t gper = (G + kThreads - 1) / kThreads;
  const int64_t g0 = min((int64_t)threadIdx.x * gper, G), g1 = min(g0 + gper, G);
  int64_t t = 0;
  for (int64_t g = g0; g < g1; ++g) t += ((offs[g + 1] - offs[g]) * upr + kTileUnits - 1) / kTileUnits;
  t = block_exclusive_scan<false>(t, &total);
  if (threadIdx.x == 0) tstart[G] = (int32_t)total;
  for (int64_t g = g0; g < g1; ++g) {
    tstart[g] = (int32_t)t;
    const int64_t tg = ((offs[g + 1] - offs[g]) * upr + kTileUnits - 1) / kTileUnits;
    if (tg == 0 && gout != nullptr) {
      gout[2 * g] = 1.0f;
      gout[2 * g + 1] = 0.0f;
    }
    t += tg;
  }
}

// table[e] = (group, tile within the group) for e < tstart[G], (-1, 0) after.
// Up to kTableLds groups the starts are searched in LDS, else in memory.
constexpr int kTableLds = 8192;
__global__ __launch_bounds__(kThreads) void tile_table_kernel(const int32_t* __restrict__ tstart,
                                                             int64_t G, int64_t entries, int2* table) {
  __shared__ int32_t st[kTableLds + 1];
  const bool in_lds = G <= kTableLds;
  if (in_lds) {
    for (int64_t i = threadIdx.x; i <= G; i += kThreads) st[i] = tstart[i];
    __syncthreads();
  }
  const int32_t* ts = in_lds ? st : tstart;
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= entries) return;
  const int32_t total = ts[G];
  if (e >= total) {
    table[e] = make_int2(-1, 0);
    return;
  }
  // last g with tstart[g] <= e (empty groups share their start with the next)
  int64_t lo = 0, hi = G - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (ts[mid] <= e) lo = mid;
    else hi = mid - 1;
  }
  table[e] = make_int2((int)lo, (int)(e - ts[lo]));
}

// Up to kMergeGroups groups, offs_prep_kernel and tile_table_kernel in one
// launch: every workgroup derives offs and tstart in LDS from the caller's
// offsets with the same two scans, workgroup 0 also stores them (and {1, 0}
// for empty groups), and each workgroup writes its kThreads table entries.
// Tiles are `tu` units. When `big` is given, workgroup 0 also stores there
// whether some group has more than big_limit tiles.
constexpr int kMergeGroups = 4096;
__global__ __launch_bounds__(kThreads) void offs_table_kernel(const int64_t* __restrict__ off_in, int64_t G,
                                                             int64_t rows, int64_t upr, int64_t entries,
                                                             int64_t* offs, int32_t* tstart, float* gout,
                                                             int2* table, int64_t tu, int32_t* big,
                                                             int64_t big_limit, int4* desc, uint32_t* zero,
                                                             int64_t zero_words) {
  __shared__ int64_t so[kMergeGroups + 1];
  __shared__ int32_t st[kMergeGroups + 1];
  const bool first = blockIdx.x == 0;
  // words to clear for the kernel that follows (the single pass's slots and S words)
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < zero_words; i += (int64_t)gridDim.x * kThreads)
    zero[i] = 0u;
  const int64_t n = G + 1;
  const int64_t per = (n + kThreads - 1) / kThreads;
  const int64_t i0 = min((int64_t)threadIdx.x * per, n), i1 = min(i0 + per, n);
  int64_t total;
  // 1. running max of the clamped offsets
  int64_t m = 0;
  for (int64_t i = i0; i < i1; ++i) m = max(m, min(max(off_in[i], (int64_t)0), rows));
  m = block_exclusive_scan<true>(m, &total);
  for (int64_t i = i0; i < i1; ++i) {
    m = max(m, min(max(off_in[i], (int64_t)0), rows));
    so[i] = m;
    if (first) offs[i] = m;
  }
  __syncthreads();
  // 2. tiles per group, exclusive prefix sum
  const int64_t gper = (G + kThreads - 1) / kThreads;
  const int64_t g0 = min((int64_t)threadIdx.x * gper, G), g1 = min(g0 + gper, G);
  int64_t t = 0, tmax = 0;
  for (int64_t g = g0; g < g1; ++g) {
    const int64_t tg = ((so[g + 1] - so[g]) * upr + tu - 1) / tu;
    t += tg;
    tmax = max(tmax, tg);
  }
  int64_t most;
  (void)block_exclusive_scan<true>(tmax, &most);
  t = block_exclusive_scan<false>(t, &total);
  if (threadIdx.x == 0) {
    st[G] = (int32_t)total;
    if (first) tstart[G] = (int32_t)total;
    if (first && big != nullptr) *big = most > big_limit ? 1 : 0;
  }
  for (int64_t g = g0; g < g1; ++g) {
    st[g] = (int32_t)t;
    const int64_t tg = ((so[g + 1] - so[g]) * upr + tu - 1) / tu;
    if (first) {
      tstart[g] = (int32_t)t;
      if (tg == 0 && gout != nullptr) {
        gout[2 * g] = 1.0f;
        gout[2 * g + 1] = 0.0f;
      }
    }
    t += tg;
  }
  __syncthreads();
  // 3. this workgroup's table entries: (group, tile within the group), or
  // with `desc` the tile descriptor {first unit (lo, hi), length, group}
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= entries) return;
  if (e >= total) {
    if (desc != nullptr) desc[e] = make_int4(0, 0, 0, -1);
    else table[e] = make_int2(-1, 0);
    return;
  }
  int64_t lo = 0, hi = G - 1;   // last g with tstart[g] <= e
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (st[mid] <= e) lo = mid;
    else hi = mid - 1;
  }
  if (desc != nullptr) {
    const int64_t base = so[lo] * upr + (e - st[lo]) * tu;
    const int64_t len = min(tu, so[lo + 1] * upr - base);
    desc[e] = make_int4((int)(uint32_t)(uint64_t)base, (int)(uint32_t)((uint64_t)base >> 32), (int)len, (int)lo);
  } else {
    table[e] = make_int2((int)lo, (int)(e - st[lo]));
  }
}

// Tile maxima of row-offset groups: tpart[e] for table entry e.
__global__ __launch_bounds__(kThreads) void tile_amax_kernel(TileMap m, const uint4* __restrict__ x,
                                                            uint32_t* tpart) {
  __shared__ uint32_t red[kThreads / 64];
  const int2 e = m.table[blockIdx.x];
  if (e.x < 0) return;
  const int64_t gbase = m.offs[e.x] * m.upr;
  const int64_t lim = m.offs[e.x + 1] * m.upr - gbase;
  const int64_t tbase = (int64_t)e.y * kTileUnits;
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < kUPT; ++j) {
    const int64_t u = tbase + j * kThreads + threadIdx.x;
    if (u < lim) mx = max(mx, unit_amax_bits(load_stream(x + gbase + u)));
  }
  mx = wave_max_u32(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) tpart[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// Guided rounding under the rollout scales (guided_fake_quant), Reconstruct
// alone (DECODE: reference codes, no y), and the fused discrepancy sums
// (STATS: SB = sum (x_t - x_r)^2 over the inputs; SF = sum (y_t - y_r)^2 with
// y_r the rollout's RTN output under the same scales, recomputed from x_r).
// Threads of a guided_kernel workgroup, whose tile is guided_tile(...) units:
// the fused statistics pass runs 256 threads (4 units each on its 1024-unit
// tile), the other modes 512 (2 units each for guided rounding, 4 for
// Reconstruct alone and row-offset groups), which
// keeps more waves per SIMD (3.7% faster for plain guided rounding of a
// streamed layer on 2048-unit tiles).
constexpr int guided_threads(bool stats) { return stats ? kThreads : 2 * kThreads; }

template <int FMT, int BITS, bool DECODE, bool WCODES, bool STATS, bool DIAG, int MAP>
__global__ __launch_bounds__(guided_threads(STATS)) void guided_kernel(GuidedArgs a) {
  constexpr int64_t TU = guided_tile(DECODE, MAP);
  constexpr int GT = guided_threads(STATS), GU = (int)(TU / GT);
  // MAP 0: one group per tile; 1: packed small groups; 2: row-offset groups.
  constexpr bool PACK = MAP == 1;
  static_assert(!(MAP == 2 && STATS), "row-offset groups take no fused statistics");
  __shared__ float2 lut[PACK ? 1 : 128];
  __shared__ float gs[PACK ? kPackGroups : 1];     // S of the tile's groups (packed)
  __shared__ uint32_t hist[DIAG ? kMismatchCounts : 1];
  int64_t g, tbase, gbase, lim;
  if constexpr (PACK) {
    g = 0;
    tbase = (int64_t)blockIdx.x * TU;
    gbase = 0;
    lim = a.map.units;
  } else if constexpr (MAP == 2) {
    const int2 e = a.map.table[blockIdx.x];
    if (e.x < 0) return;
    g = e.x;
    tbase = (int64_t)e.y * TU;
    gbase = a.map.offs[g] * a.map.upr;
    lim = a.map.offs[g + 1] * a.map.upr - gbase;
  } else {
    tile_of(a.map, g, tbase);
    gbase = g * a.map.upg;
    lim = a.map.upg;
  }
  if constexpr (DIAG) {
    if (threadIdx.x < kMismatchCounts) hist[threadIdx.x] = 0u;
  }
  if constexpr (STATS) {
    if (a.ticket != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
      __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The fused statistics pass over equal groups and the row-offset passes,
  // with no record or a 1-bit one (WRUN): each wave takes 64 * GU
  // consecutive units (unit j of lane l at j * 64 + l), so the wave's scale
  // bytes (one per block: two units for NVFP4, four for MXFP4) and record
  // bytes (one per unit) are one contiguous run each. A wave whose runs lie
  // inside the group and start on a dword reads them as one dword per lane
  // and hands each lane its bytes with ds_bpermute (two loads per lane
  // instead of two per unit); any other wave reads them per unit. The x, x_r
  // and y accesses stay one contiguous KiB per wave instruction either way.
  // Elsewhere unit j of thread t is at j * GT + t: there this layout measured
  // slower (plain guided rounding by 0.6%, 2- and 3-bit records by 2-6%).
  constexpr bool WRUN = ((STATS && MAP == 0) || MAP == 2) && BITS <= 1;
  constexpr int SU = FMT == 0 ? 1 : 2;   // log2 of the units per block
  const int wl = (int)threadIdx.x & 63;
  const int64_t wb = tbase + (int64_t)((int)threadIdx.x >> 6) * (GU * 64);   // the wave's first unit (WRUN)
  bool words = false;
  uint32_t sdw = 0u, gdw = 0u;
  if constexpr (WRUN) {
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(a.scales + ((gbase + wb) >> SU));
    const uint32_t* gp = BITS == 1 ? reinterpret_cast<const uint32_t*>(a.guide + gbase + wb) : nullptr;
    words = wb + GU * 64 <= lim && (reinterpret_cast<uintptr_t>(sp) & 3u) == 0 &&
            (reinterpret_cast<uintptr_t>(gp) & 3u) == 0;
    if (words) {
      if (wl < (16 >> SU) * GU) sdw = __builtin_nontemporal_load(sp + wl);
      if (BITS == 1 && wl < 16 * GU) gdw = __builtin_nontemporal_load(gp + wl);
    }
  }
  // Issue the tile's loads first; the factor table is built while they fly.
  uint4 v[GU];
  uint4 vr[STATS ? GU : 1];
  uint32_t sbv[GU], gv[GU];
#pragma unroll
  for (int j = 0; j < GU; ++j) {
    const int64_t u = WRUN ? wb + j * 64 + wl : tbase + j * GT + threadIdx.x;
    const bool ok = u < lim;
    const int64_t gu = gbase + u;
    v[j] = ok ? load_stream(a.x + gu) : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (STATS) vr[j] = ok ? load_stream(a.xr + gu) : make_uint4(0u, 0u, 0u, 0u);
    sbv[j] = 0u;
    gv[j] = 0u;
    if (WRUN && words) {
      if constexpr (BITS <= 1) continue;   // scale and record bytes from the dwords below
    } else {
      sbv[j] = ok ? (uint32_t)__builtin_nontemporal_load(a.scales + (FMT == 0 ? (gu >> 1) : (gu >> 2))) : 0u;
      if constexpr (BITS == 1) gv[j] = ok ? (uint32_t)__builtin_nontemporal_load(a.guide + gu) : 0u;
    }
    if constexpr (BITS == 2) {
      gv[j] = ok ? (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(a.guide) + gu) : 0u;
    } else if constexpr (BITS == 3) {
      const uint8_t* q = a.guide + 3 * gu;
      gv[j] = ok ? (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) : 0u;
    } else if constexpr (BITS == 4) {
      gv[j] = ok ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.guide) + gu) : 0u;
    }
  }
  if constexpr (WRUN) {
    if (words) {   // uniform in the wave, so every lane takes part in the permutes
#pragma unroll
      for (int j = 0; j < GU; ++j) {
        // unit o = j * 64 + wl of the run: scale byte o >> SU, record byte o
        const uint32_t sw = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (j * (16 >> SU) + (wl >> (SU + 2))), (int)sdw);
        sbv[j] = (sw >> (8 * ((wl >> SU) & 3))) & 0xFFu;
        if constexpr (BITS == 1) {
          const uint32_t gw = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (j * 16 + (wl >> 2)), (int)gdw);
          gv[j] = (gw >> (8 * (wl & 3))) & 0xFFu;
        }
      }
    }
  }
  if constexpr (PACK) {
    const int64_t g0t = tbase >> a.map.lg;
    for (int i = threadIdx.x; i < (TU >> a.map.lg); i += GT) {
      const int64_t gg = g0t + i;
      gs[i] = gg < a.map.groups ? a.gscale[2 * gg] : 1.0f;
    }
  } else if constexpr (FMT == 0) {
    build_factor_lut(lut, a.gscale[2 * g]);
  }
  if constexpr (FMT == 0 || DIAG) __syncthreads();
  double acc_b = 0.0, acc_f = 0.0;
#pragma unroll
  for (int j = 0; j < GU; ++j) {
    const int64_t u = WRUN ? wb + j * 64 + wl : tbase + j * GT + threadIdx.x;
    float r, d = 0.0f, dsc = 0.0f;
    if constexpr (PACK) {
      nv_factors_pair(sbv[j], gs[(j * GT + threadIdx.x) >> a.map.lg], r, d);
    } else if constexpr (FMT == 0) {
      const float2 rd = lut[sbv[j] & 0x7Fu];
      r = rd.x;
      d = rd.y;
    } else {
      r = mx_r(sbv[j]);
      dsc = mx_dscale(sbv[j]);
    }
    float f[8], t[8];
    unit_f32(v[j], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = f[i] * r;
    const uint32_t K = select_codes<BITS, DECODE>(t, gv[j]);
    uint4 yv = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (!DECODE) yv = FMT == 0 ? dequant_nv(K, d) : dequant_mx(K, dsc);
    if constexpr (STATS) {
      float fr[8];
      unit_f32(vr[j], fr);
      acc_b += sq_diff_sum(f, fr);
#pragma unroll
      for (int i = 0; i < 8; ++i) fr[i] *= r;
      const uint32_t KR = rtn_codes(fr);
      if (K != KR) {  // equal codes under one scale give equal outputs
        const uint4 yr = FMT == 0 ? dequant_nv(KR, d) : dequant_mx(KR, dsc);
        float ft[8], fq[8];
        unit_f32(yv, ft);
        unit_f32(yr, fq);
        acc_f += sq_diff_sum(ft, fq);
      }
      if constexpr (DIAG) {
        const uint32_t K0 = BITS == 0 ? K : rtn_codes(t);
        if (u < lim && (K != KR || K0 != KR)) mismatch_unit(K, KR, K0, hist);
      }
    }
    if (u < lim) {
      const int64_t gu = gbase + u;
      if constexpr (DECODE || WCODES) __builtin_nontemporal_store(K, a.codes + gu);
      if constexpr (!DECODE) store_stream(a.y + gu, yv);
    }
  }
  if constexpr (STATS) {
    group_sum2<GT>(acc_b, acc_f);
    if (threadIdx.x == 0) {
      a.partials[2 * blockIdx.x] = acc_b;
      a.partials[2 * blockIdx.x + 1] = acc_f;
    }
  }
  if constexpr (DIAG) {
    __syncthreads();
    if (threadIdx.x < kMismatchCounts) {
      // Distance 0 (bins 0 and 15) is the rest of the tile's elements.
      const int64_t valid = min(TU, lim - tbase) * kUnitElems;
      const int b = threadIdx.x;
      uint32_t hv = hist[b];
      if (b == 0 || b == kMismatchBins) {
        uint32_t others = 0;
        for (int i = 1; i < kMismatchBins; ++i) others += hist[b + i];
        hv = (uint32_t)valid - others;
      }
      a.cpart[(int64_t)b * gridDim.x + blockIdx.x] = hv;
    }
  }
}

// Sums the per-tile mismatch counts of bin blockIdx.x into counts (int64).
__global__ __launch_bounds__(kThreads) void counts_final_kernel(const uint32_t* __restrict__ cpart,
                                                                int64_t tiles, int64_t* counts,
                                                                int accumulate) {
  const uint32_t* p = cpart + (int64_t)blockIdx.x * tiles;
  unsigned long long s = 0;
  for (int64_t i = threadIdx.x; i < tiles; i += kThreads) s += p[i];
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  __shared__ unsigned long long ws[kThreads / 64];
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t += ws[w];
    if (accumulate) counts[blockIdx.x] += (int64_t)t;
    else counts[blockIdx.x] = (int64_t)t;
  }
}

// First level of the partial-sum reduction: workgroup w sums pairs
// [w*per, min((w+1)*per, count)) of `in` into out[w] (fixed order).
__global__ __launch_bounds__(kThreads) void sums_mid_kernel(const double* __restrict__ in,
                                                            int64_t count, int64_t per,
                                                            double* __restrict__ out) {
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = min(lo + per, count);
  double sb = 0.0, sf = 0.0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) {
    sb += in[2 * i];
    sf += in[2 * i + 1];
  }
  group_sum2(sb, sf);
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = sb;
    out[2 * blockIdx.x + 1] = sf;
  }
}

// Fixed-order reduction of `groups` partial pairs into acc3 = {SB, SF, n}, by
// one workgroup of kSumThreads. Thread t sums pairs t, t + kSumThreads, ... in
// order, loading kSumBatch pairs at a time (two round trips to memory for
// 34 pairs per thread); the 16 wave sums are then added in wave order.
// (Workspaces are only 8-byte aligned: a pair is two loads.)
constexpr int kSumThreads = 1024;
constexpr int kSumBatch = 17;

// This thread's share of pairs [lo, hi): lo + t, lo + t + kSumThreads, ...
__device__ __forceinline__ void pair_range_sum(const double* __restrict__ p, int64_t lo, int64_t hi, double& sb,
                                               double& sf) {
  for (int64_t base = lo + threadIdx.x; base < hi; base += (int64_t)kSumBatch * kSumThreads) {
    double2 v[kSumBatch];
#pragma unroll
    for (int k = 0; k < kSumBatch; ++k) {
      const int64_t i = base + (int64_t)k * kSumThreads;
      v[k] = i < hi ? make_double2(p[2 * i], p[2 * i + 1]) : make_double2(0.0, 0.0);
    }
#pragma unroll
    for (int k = 0; k < kSumBatch; ++k) {
      sb += v[k].x;
      sf += v[k].y;
    }
  }
}

// The kSumThreads threads' sums added in wave order; valid in thread 0.
__device__ __forceinline__ void pair_block_sum(double& sb, double& sf) {
  __shared__ double wb[kSumThreads / 64], wf[kSumThreads / 64];
  sb = wave_sum(sb);
  sf = wave_sum(sf);
  if ((threadIdx.x & 63) == 0) {
    wb[threadIdx.x >> 6] = sb;
    wf[threadIdx.x >> 6] = sf;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    sb = wb[0];
    sf = wf[0];
    for (int w = 1; w < kSumThreads / 64; ++w) {
      sb += wb[w];
      sf += wf[w];
    }
  }
}

__device__ __forceinline__ void put_acc3(double* acc3, double sb, double sf, int64_t n, int accumulate) {
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

__global__ __launch_bounds__(kSumThreads) void sums_final_kernel(const double* __restrict__ partials,
                                                                 int64_t groups, int64_t n, double* acc3,
                                                                 int accumulate) {
  double sb = 0.0, sf = 0.0;
  pair_range_sum(partials, 0, groups, sb, sf);
  pair_block_sum(sb, sf);
  if (threadIdx.x == 0) put_acc3(acc3, sb, sf, n, accumulate);
}

// The same reduction over kSplitGroups workgroups, one per XCD, for the
// fused pass's per-tile pairs (one workgroup reads them at one CU's rate:
// 7.6 µs for a streamed layer's 34,816; eight take 5.7). Workgroup w sums pairs
// [w * per, (w + 1) * per) as above and stores its pair to mid[w] with
// agent-scope stores; once they are complete it takes a ticket from an
// agent-scope counter that the guided kernel zeroed, and the workgroup with
// the last ticket adds the kSplitGroups pairs in index order into acc3. The
// result does not depend on which workgroup finishes last; nothing waits.
constexpr int kSplitGroups = 8;
constexpr int64_t kSplitMin = 8192;   // pairs from which the final sum is split
static_assert(2 * kSplitGroups < 2 * kMidGroups - 1, "the split pairs and the counter fit the second-level area");
__global__ __launch_bounds__(kSumThreads) void sums_split_kernel(const double* __restrict__ partials, int64_t count,
                                                                 int64_t per, double* mid, uint32_t* ticket,
                                                                 int64_t n, double* acc3, int accumulate) {
  const int64_t lo = min((int64_t)blockIdx.x * per, count), hi = min(lo + per, count);
  double sb = 0.0, sf = 0.0;
  pair_range_sum(partials, lo, hi, sb, sf);
  pair_block_sum(sb, sf);
  if (threadIdx.x != 0) return;
  __hip_atomic_store(&mid[2 * blockIdx.x], sb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&mid[2 * blockIdx.x + 1], sf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);   // the pair is stored before the ticket is taken
  const uint32_t t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t != gridDim.x - 1) return;
  double ab = 0.0, af = 0.0;
  for (int w = 0; w < (int)gridDim.x; ++w) {
    ab += __hip_atomic_load(&mid[2 * w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    af += __hip_atomic_load(&mid[2 * w + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  put_acc3(acc3, ab, af, n, accumulate);
}

// ------------------------------------------------------------ discrepancy_stats

__device__ __forceinline__ void accum_unit(const uint4& a, const uint4& b, double& acc) {
  float fa[8], fb[8];
  unit_f32(a, fa);
  unit_f32(b, fb);
  acc += sq_diff_sum(fa, fb);
}

__device__ __forceinline__ double bf16_f64(uint32_t b) { return (double)__uint_as_float(b << 16); }

constexpr int kStatsUnits = 4;   // units per thread and array in a discrepancy_stats tile
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
  // Workgroup tiles of kStatsUnits * kThreads consecutive units (unit k of
  // thread t at k * kThreads + t), the workgroups striding over the arrays
  // tile by tile; every load of a tile is issued before its sums. Against
  // one unit per thread and stride: 337 against 370 µs for four arrays of a
  // streamed layer (84% of the HBM peak against 77%); 6 or 8 units tie.
  double sb = 0.0, sf = 0.0;
  const int64_t tstride = (int64_t)gridDim.x * kThreads * kStatsUnits;
  for (int64_t tb = (int64_t)blockIdx.x * kThreads * kStatsUnits; tb < units; tb += tstride) {
    uint4 a[kStatsUnits], b[kStatsUnits], c[kStatsUnits], d[kStatsUnits];
#pragma unroll
    for (int k = 0; k < kStatsUnits; ++k) {
      const int64_t u = tb + k * kThreads + threadIdx.x;
      const bool ok = u < units;
      a[k] = ok ? load_stream(xt4 + u) : make_uint4(0u, 0u, 0u, 0u);
      b[k] = ok ? load_stream(xr4 + u) : make_uint4(0u, 0u, 0u, 0u);
      c[k] = ok ? load_stream(yt4 + u) : make_uint4(0u, 0u, 0u, 0u);
      d[k] = ok ? load_stream(yr4 + u) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kStatsUnits; ++k) {   // zero units add nothing
      accum_unit(a[k], b[k], sb);
      accum_unit(c[k], d[k], sf);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int64_t i = units * kUnitElems; i < n; ++i) {
      const double dx = bf16_f64(xt[i]) - bf16_f64(xr[i]);
      const double dy = bf16_f64(yt[i]) - bf16_f64(yr[i]);
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

// MXFP4 has no global scale, so a call's groups are one tensor to it.
Shape effective(int fmt, const Shape& sh) {
  if (fmt == 1 && sh.groups > 1) return Shape{1, sh.groups * sh.upg};
  return sh;
}

// NVFP4 groups whose unit count is a power of two below a tile are packed
// several to a tile (and their encode reads the input once).
bool packable(int fmt, const Shape& sh, int64_t tu = kTileUnits) {
  return fmt == 0 && sh.groups > 1 && sh.upg > 0 && sh.upg < tu && tu % sh.upg == 0;
}

TileMap tile_map(int fmt, const Shape& sh0, int64_t tu = kTileUnits) {
  const Shape sh = effective(fmt, sh0);
  TileMap m{};
  m.tu = tu;
  m.upg = sh.upg;
  m.units = sh.groups * sh.upg;
  m.groups = sh.groups;
  if (packable(fmt, sh, tu)) {
    m.tiles = (m.units + tu - 1) / tu;
    m.lg = __builtin_ctzll((unsigned long long)sh.upg);
    m.packed = 1;
  } else {
    m.tiles = (sh.upg + tu - 1) / tu;
  }
  return m;
}

int64_t tile_grid(const TileMap& m) { return m.packed ? m.tiles : m.groups * m.tiles; }

std::atomic<int64_t> g_encode_batch{0};   // groups per batch; 0 = automatic (kCacheBatchBytes of input)
std::atomic<int64_t> g_wait_limit{0};     // polls per bounded wait; 0 = kSpinMax
constexpr int64_t kCacheBatchBytes = (int64_t)96 << 20;

int amax_parts(int64_t upg) {
  int64_t p = (upg + (int64_t)kThreads * 8 - 1) / ((int64_t)kThreads * 8);
  if (p < 1) p = 1;
  if (p > kPartMax) p = kPartMax;
  return (int)p;
}

template <int FMT, int PLANE, bool WY, int SSRC, bool PACK>
hipError_t quant_go(const QuantArgs& a, int64_t blocks, hipStream_t s) {
  return launch(quantize_kernel<FMT, PLANE, WY, SSRC, PACK>, dim3((unsigned)blocks),
                dim3(quant_threads(SSRC, PACK)), s, a);
}

// `blocks`: the launch's workgroups (quantize tiles, then side amax work).
// ssrc: 0 S given, 1 S from amax partials, 2 S from the tile's own groups
// (packed), 3 S from the tile maxima of row-offset groups.
template <int FMT, int PLANE, bool WY>
hipError_t quant_src(int ssrc, bool pack, const QuantArgs& a, int64_t blocks, hipStream_t s) {
  if constexpr (FMT == 1) {
    return quant_go<1, PLANE, WY, 0, false>(a, blocks, s);
  } else {
    if (pack) return ssrc ? quant_go<0, PLANE, WY, 2, true>(a, blocks, s)
                          : quant_go<0, PLANE, WY, 0, true>(a, blocks, s);
    if (ssrc == 3) return quant_go<0, PLANE, WY, 3, false>(a, blocks, s);
    return ssrc ? quant_go<0, PLANE, WY, 1, false>(a, blocks, s)
                : quant_go<0, PLANE, WY, 0, false>(a, blocks, s);
  }
}

template <int FMT, int PLANE>
hipError_t quant_wy(bool wy, int ssrc, bool pack, const QuantArgs& a, int64_t blocks, hipStream_t s) {
  return wy ? quant_src<FMT, PLANE, true>(ssrc, pack, a, blocks, s)
            : quant_src<FMT, PLANE, false>(ssrc, pack, a, blocks, s);
}

// plane_mode = bits of the guidance plane (1..4; quantize_rtn writes codes, 4).
template <int FMT>
hipError_t quant_plane(int plane_mode, bool wy, int ssrc, bool pack, const QuantArgs& a,
                       int64_t blocks, hipStream_t s) {
  switch (plane_mode) {
    case 1: return quant_wy<FMT, 1>(wy, ssrc, pack, a, blocks, s);
    case 2: return quant_wy<FMT, 2>(wy, ssrc, pack, a, blocks, s);
    case 3: return quant_wy<FMT, 3>(wy, ssrc, pack, a, blocks, s);
    default: return quant_wy<FMT, 4>(wy, ssrc, pack, a, blocks, s);
  }
}

// ---- single-pass encode (onepass_encode_kernel)

constexpr int kOnePassTiles = kPartMax;  // most tiles per group (slot layout); the grid bounds it further
constexpr int kOnePassPerCU = 2;         // resident workgroups per CU it is built for

template <int PLANE, bool WY>
const void* onepass_fn(bool table) {
  return table ? reinterpret_cast<const void*>(&onepass_encode_kernel<PLANE, WY, true>)
               : reinterpret_cast<const void*>(&onepass_encode_kernel<PLANE, WY, false>);
}

const void* onepass_kernel(int plane_mode, bool wy, bool table) {
  switch (plane_mode) {
    case 1: return wy ? onepass_fn<1, true>(table) : onepass_fn<1, false>(table);
    case 2: return wy ? onepass_fn<2, true>(table) : onepass_fn<2, false>(table);
    case 3: return wy ? onepass_fn<3, true>(table) : onepass_fn<3, false>(table);
    default: return wy ? onepass_fn<4, true>(table) : onepass_fn<4, false>(table);
  }
}

// Workgroups that may be resident at once for the kernel: kOnePassPerCU per
// CU if the occupancy query allows that many, else 0 (not used). Cached per
// device and kernel.
int64_t onepass_capacity(const void* k, int dev) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int64_t> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({dev, k});
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  int64_t cap = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k, kOnePassThreads, 0) == hipSuccess &&
      per >= kOnePassPerCU)
    cap = (int64_t)cus * kOnePassPerCU;
  cache[{dev, k}] = cap;
  return cap;
}

// Single-pass launches of one process on one device run one after another,
// whatever their streams: each needs the whole device resident at once, so
// two running side by side could each hold part of it and wait on the other
// (the bounded waits end that, through the slow exact path). While every
// launch comes on one stream, stream order suffices and nothing is added (an
// event per launch costs ~7 us of the next kernel's start). The first launch
// on another stream is ordered after the previous launch by an event recorded
// on that launch's stream at that moment; from then on each launch records
// its own event and the next launch on another stream waits for it. No host
// synchronization is involved. Nothing is done while the stream is being
// captured into a graph (a graph runs its nodes in order).
struct OnePassOrder {
  std::mutex mu;
  hipEvent_t ev = nullptr;     // created once per device, with the device's symbols
  bool multi = false;          // launches seen on more than one stream
  bool recorded = false;       // ev holds the last launch (multi mode)
  bool any = false;            // a launch happened
  hipStream_t last = nullptr;  // stream of the last launch
};
OnePassOrder g_onepass_order[64];

// Per-device set-up, done once with the device current: the device addresses
// of the library's device variables, and the single-pass ordering event (so
// no call allocates or creates anything afterwards).
struct DeviceSyms {
  bool ready = false;
  unsigned long long* fails = nullptr;
  uint8_t* scratch = nullptr;
};
std::mutex g_syms_mu;
DeviceSyms g_syms[64];

hipError_t device_syms(int dev, const DeviceSyms** out) {
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_syms_mu);
  DeviceSyms& d = g_syms[dev];
  if (!d.ready) {
    void* p = nullptr;
    void* q = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_wait_fails));
    if (e != hipSuccess) return e;
    if ((e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    OnePassOrder& ord = g_onepass_order[dev];
    {
      std::lock_guard<std::mutex> olock(ord.mu);
      if (ord.ev == nullptr && (e = hipEventCreateWithFlags(&ord.ev, hipEventDisableTiming)) != hipSuccess)
        return e;
    }
    d.fails = static_cast<unsigned long long*>(p);
    d.scratch = static_cast<uint8_t*>(q);
    d.ready = true;
  }
  *out = &d;
  return hipSuccess;
}

// Enqueues a single-pass launch: orders it after the device's previous one
// (see OnePassOrder), clears its `words` words of slots and S words at
// `zero` with a fill kernel when words > 0 (no memset, so the call can be
// captured in a graph), then launches `grid` workgroups of kernel k with
// arguments a.
hipError_t onepass_enqueue(const void* k, OnePassArgs& a, int64_t grid, uint32_t* zero, int64_t words, int dev,
                           const DeviceSyms* syms, hipStream_t stream) {
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &capture);
  if (e != hipSuccess) return e;
  OnePassOrder& ord = g_onepass_order[dev];
  std::unique_lock<std::mutex> lock(ord.mu, std::defer_lock);
  if (capture == hipStreamCaptureStatusNone) {
    lock.lock();
    if (ord.any && ord.last != stream && !ord.multi) {
      // first launch on a second stream: the previous launch left no event,
      // so one is recorded now on its stream (after everything enqueued there)
      if ((e = hipEventRecord(ord.ev, ord.last)) != hipSuccess) return e;
      ord.multi = true;
      ord.recorded = true;
    }
    if (ord.multi && ord.recorded && ord.last != stream && (e = hipStreamWaitEvent(stream, ord.ev, 0)) != hipSuccess)
      return e;
  }
  a.fails = syms->fails;
  const int64_t wl = g_wait_limit.load(std::memory_order_relaxed);
  a.spin_max = wl > 0 ? (int)wl : kSpinMax;
  if (words > 0) {
    const int64_t zb = min((words + kThreads - 1) / kThreads, (int64_t)1024);
    e = launch(zero_words_kernel, dim3((unsigned)zb), dim3(kThreads), stream, zero, words);
    if (e != hipSuccess) return e;
  }
  // An ordinary launch on the caller's queue: the grid is at most the
  // resident capacity, and the workgroups wait only for each other, so every
  // one of them becomes resident once earlier work on the device drains (a
  // cooperative launch would guarantee the same but goes through another
  // hardware queue, ~11 us of switching before and after the kernel).
  void* argv[] = {&a};
  e = hipLaunchKernel(k, dim3((unsigned)grid), dim3(kOnePassThreads), argv, 0, stream);
  if (e != hipSuccess) return e;
  if (capture == hipStreamCaptureStatusNone) {
    if (ord.multi) {
      if ((e = hipEventRecord(ord.ev, stream)) != hipSuccess) return e;
      ord.recorded = true;
    }
    ord.any = true;
    ord.last = stream;
  }
  return hipSuccess;
}

// Launches the single-pass encode of equal groups when it applies; *used
// tells whether it did.
hipError_t launch_onepass(int plane_mode, bool wy, const Shape& sh, const QuantArgs& qa, void* work,
                          hipStream_t stream, bool* used) {
  *used = false;
  const int64_t Tmin = (sh.upg + kOPTile - 1) / kOPTile;
  if (Tmin > kOnePassTiles) return hipSuccess;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipSuccess;
  const void* k = onepass_kernel(plane_mode, wy, false);
  const int64_t cap = onepass_capacity(k, dev);
  const int64_t Q = min(sh.groups, (cap - 1) / Tmin);   // + the combining workgroup
  // the kernel indexes groups with 32-bit ints, up to groups + 4Q
  if (Q < 1 || sh.groups + 5 * Q > INT32_MAX) return hipSuccess;
  // Spread each group over as many tiles as the resident grid allows (equal
  // work per CU), in multiples of 64 units: a wave's plane and y stores then
  // start on whole 64-byte segments, and no NVFP4 block straddles two tiles.
  const int64_t Tfit = min((cap - 1) / Q, (int64_t)kOnePassTiles);
  const int64_t L = ((sh.upg + Tfit - 1) / Tfit + 63) / 64 * 64;
  const int64_t T = (sh.upg + L - 1) / L;
  const DeviceSyms* syms = nullptr;
  hipError_t e = device_syms(dev, &syms);
  if (e != hipSuccess) return e;
  OnePassArgs a{};
  a.x = qa.x;
  a.upg = (int)sh.upg;
  a.groups = (int)sh.groups;
  a.T = (int)T;
  a.Q = (int)Q;
  a.L = (int)L;
  a.copies = kSCopies;
  a.slots = static_cast<uint32_t*>(work);
  a.sword = a.slots + sh.groups * kPartMax;
  a.gout = qa.gout;
  a.plane = qa.plane;
  a.scales = qa.scales;
  a.y = qa.y;
  e = onepass_enqueue(k, a, Q * T + 1, a.slots, sh.groups * ((int64_t)kPartMax + kSCopies * 64), dev, syms, stream);
  if (e == hipSuccess) *used = true;
  return e;
}

template <int FMT, int BITS, bool DECODE, bool WCODES, bool STATS, bool DIAG, int MAP>
hipError_t guided_go(const GuidedArgs& a, int64_t blocks, hipStream_t s) {
  return launch(guided_kernel<FMT, BITS, DECODE, WCODES, STATS, DIAG, MAP>, dim3((unsigned)blocks),
                dim3(guided_threads(STATS)), s, a);
}

template <int FMT, int BITS, int MAP>
hipError_t guided_bits(bool wc, bool stats, bool diag, const GuidedArgs& a, int64_t blocks,
                       hipStream_t s) {
  if constexpr (MAP != 2) {
    if (diag) return wc ? guided_go<FMT, BITS, false, true, true, true, MAP>(a, blocks, s)
                        : guided_go<FMT, BITS, false, false, true, true, MAP>(a, blocks, s);
    if (stats) return wc ? guided_go<FMT, BITS, false, true, true, false, MAP>(a, blocks, s)
                         : guided_go<FMT, BITS, false, false, true, false, MAP>(a, blocks, s);
  }
  return wc ? guided_go<FMT, BITS, false, true, false, false, MAP>(a, blocks, s)
            : guided_go<FMT, BITS, false, false, false, false, MAP>(a, blocks, s);
}

template <int FMT, int MAP>
hipError_t guided_pack(int bits, bool decode, bool wc, bool stats, bool diag, const GuidedArgs& a,
                       int64_t blocks, hipStream_t s) {
  if (decode) {
    switch (bits) {
      case 1: return guided_go<FMT, 1, true, true, false, false, MAP>(a, blocks, s);
      case 2: return guided_go<FMT, 2, true, true, false, false, MAP>(a, blocks, s);
      default: return guided_go<FMT, 3, true, true, false, false, MAP>(a, blocks, s);
    }
  }
  switch (bits) {
    case 0: return guided_bits<FMT, 0, MAP>(wc, stats, diag, a, blocks, s);
    case 1: return guided_bits<FMT, 1, MAP>(wc, stats, diag, a, blocks, s);
    case 2: return guided_bits<FMT, 2, MAP>(wc, stats, diag, a, blocks, s);
    case 3: return guided_bits<FMT, 3, MAP>(wc, stats, diag, a, blocks, s);
    default: return guided_bits<FMT, 4, MAP>(wc, stats, diag, a, blocks, s);
  }
}

}  // namespace

int64_t quant_work_bytes(int fmt, const Shape& sh) {
  if (fmt != 0 || packable(fmt, sh)) return 0;
  // amax partials or tagged tile maxima [G][kPartMax], S words [G][kSCopies * 64]
  const int64_t words = sh.groups * ((int64_t)kPartMax + kSCopies * 64);
  return (words * (int64_t)sizeof(uint32_t) + 7) / 8 * 8;
}

int64_t guided_stats_work_bytes(int fmt, const Shape& sh) {
  // sized for the smaller tile, whose count is never below the other's
  const int64_t tiles = tile_grid(tile_map(fmt, sh, kGuidedTileUnits));
  return 2 * (int64_t)sizeof(double) * (tiles + kMidGroups) +
         (int64_t)sizeof(uint32_t) * kMismatchCounts * tiles;
}

int64_t stats_groups(int64_t n) {
  int64_t units = n / kUnitElems;
  int64_t g = (units + (int64_t)kThreads * kStatsUnits - 1) / ((int64_t)kThreads * kStatsUnits);   // tiles
  if (g < 1) g = 1;
  if (g > 1024) g = 1024;
  return g;
}

int64_t stats_work_bytes(int64_t n) { return 2 * (int64_t)sizeof(double) * stats_groups(n); }

hipError_t launch_quantize(int fmt, int plane_mode, const Shape& sh, const uint16_t* x,
                           const float* gin, float* gout, uint8_t* plane, uint8_t* scales,
                           uint16_t* y, void* work, hipStream_t stream) {
  const int64_t units = sh.groups * sh.upg;
  if (units == 0) {
    if (gout == nullptr || sh.groups == 0) return hipSuccess;
    return launch(fill_gscale_kernel, dim3((unsigned)((sh.groups + 63) / 64)), dim3(64), stream, gout,
                  sh.groups);
  }
  QuantArgs a{};
  a.map = tile_map(fmt, sh);
  a.x = reinterpret_cast<const uint4*>(x);
  a.gin = gin;
  a.gout = gout;
  a.plane = plane;
  a.scales = scales;
  a.y = reinterpret_cast<uint4*>(y);
  const bool wy = y != nullptr;
  if (a.map.packed) {  // one pass: every group's amax is reduced inside its tile
    a.qblocks = a.map.tiles;
    return quant_plane<0>(plane_mode, wy, gout != nullptr ? 2 : 0, true, a, a.qblocks, stream);
  }
  if (fmt == 1 || gout == nullptr) {
    a.qblocks = tile_grid(a.map);
    if (fmt == 0) return quant_plane<0>(plane_mode, wy, 0, false, a, a.qblocks, stream);
    return quant_plane<1>(plane_mode, wy, 0, false, a, a.qblocks, stream);
  }
  // NVFP4 with S from the amax. Calls of two or more groups of at most
  // kOnePassTiles tiles are encoded in one pass (unless a batch size was
  // set); otherwise the input is read twice (amax, then quantize). A single
  // group has nothing to overlap its combine and its last quantize with, and
  // two launches are faster there (an 8192 x 2048 chunk: 17.9 against 24.3
  // us; from two groups on the single pass wins: 30.0 against 32.6 us).
  if (g_encode_batch.load(std::memory_order_relaxed) == 0 && sh.groups >= 2) {
    bool used = false;
    hipError_t e1 = launch_onepass(plane_mode, wy, sh, a, work, stream, &used);
    if (e1 != hipSuccess || used) return e1;
  }
  // Two passes: groups go in batches of about kCacheBatchBytes of input, and
  // the launch that quantizes batch b also runs the amax pass of batch b + 1,
  // so each batch is re-read one launch after its first read. (On MI355X the
  // re-read runs at the plain HBM rate, not from the Infinity Cache, for any
  // batch size measured.) A caller-set batch size overrides the automatic one
  // (trace_set_encode_batch).
  AmaxArgs m{};
  m.x = a.x;
  m.upg = sh.upg;
  m.nparts = amax_parts(sh.upg);
  m.part = static_cast<uint32_t*>(work);
  a.part = m.part;
  a.nparts = m.nparts;
  const int64_t gbytes = sh.upg * (int64_t)sizeof(uint4);
  int64_t bg = g_encode_batch.load(std::memory_order_relaxed);
  if (bg == 0) bg = kCacheBatchBytes / (gbytes > 0 ? gbytes : 1);
  if (bg < 1) bg = 1;
  if (bg > sh.groups) bg = sh.groups;
  m.g0 = 0;
  hipError_t e = launch(amax_kernel, dim3((unsigned)(bg * m.nparts)), dim3(kThreads), stream, m);
  for (int64_t g0 = 0; e == hipSuccess && g0 < sh.groups; g0 += bg) {
    const int64_t nq = min(bg, sh.groups - g0);
    const int64_t rest = sh.groups - g0 - nq;
    const int64_t na = rest < bg ? rest : bg;
    a.g0 = g0;
    a.qblocks = nq * a.map.tiles;
    a.side = m;
    a.side.g0 = g0 + nq;
    const int64_t blocks = a.qblocks + na * m.nparts;
    e = quant_plane<0>(plane_mode, wy, 1, false, a, blocks, stream);
  }
  return e;
}

hipError_t launch_guided(int fmt, int bits, bool decode_only, const Shape& sh, const uint16_t* x,
                         const uint8_t* guide, const uint8_t* scales, const float* gscale,
                         uint16_t* y, uint8_t* codes, const uint16_t* xr, double* acc3,
                         int64_t* counts, int accumulate, void* work, hipStream_t stream) {
  const int64_t units = sh.groups * sh.upg;
  const bool stats = acc3 != nullptr;
  const bool diag = stats && counts != nullptr;
  if (units == 0) {
    if (!stats) return hipSuccess;
    hipError_t e = launch(sums_final_kernel, dim3(1), dim3(kSumThreads), stream, (const double*)nullptr,
                          (int64_t)0, (int64_t)0, acc3, accumulate);
    if (e != hipSuccess || !diag) return e;
    return launch(counts_final_kernel, dim3(kMismatchCounts), dim3(kThreads), stream,
                  (const uint32_t*)nullptr, (int64_t)0, counts, accumulate);
  }
  GuidedArgs a{};
  a.map = tile_map(fmt, sh, guided_tile(decode_only, 0));
  a.x = reinterpret_cast<const uint4*>(x);
  a.guide = guide;
  a.scales = scales;
  a.gscale = gscale;
  a.y = reinterpret_cast<uint4*>(y);
  a.codes = reinterpret_cast<uint32_t*>(codes);
  a.xr = reinterpret_cast<const uint4*>(xr);
  a.partials = static_cast<double*>(work);
  const int64_t tiles = tile_grid(a.map);
  if (stats) a.cpart = reinterpret_cast<uint32_t*>(a.partials + 2 * (tiles + kMidGroups));
  // The split final sum keeps its pairs and counter in the second-level area
  // (unused below kDirectTiles): pairs at [0, kSplitGroups), the counter in
  // the area's last word.
  const bool split = stats && tiles >= kSplitMin && tiles <= kDirectTiles;
  if (split) a.ticket = reinterpret_cast<uint32_t*>(a.partials + 2 * (tiles + kMidGroups) - 1);
  const bool wc = codes != nullptr;
  hipError_t e;
  if (fmt == 1) e = guided_pack<1, 0>(bits, decode_only, wc, stats, diag, a, tiles, stream);
  else if (a.map.packed) e = guided_pack<0, 1>(bits, decode_only, wc, stats, diag, a, tiles, stream);
  else e = guided_pack<0, 0>(bits, decode_only, wc, stats, diag, a, tiles, stream);
  if (e != hipSuccess || !stats) return e;
  if (diag) {
    e = launch(counts_final_kernel, dim3(kMismatchCounts), dim3(kThreads), stream,
               (const uint32_t*)a.cpart, tiles, counts, accumulate);
    if (e != hipSuccess) return e;
  }
  // Per-tile pairs -> acc3 in one workgroup (below kSplitMin pairs), in
  // kSplitGroups workgroups (up to kDirectTiles), else per-tile pairs ->
  // kMidGroups pairs -> acc3; each level in a fixed order.
  if (split) {
    const int64_t per = (tiles + kSplitGroups - 1) / kSplitGroups;
    return launch(sums_split_kernel, dim3(kSplitGroups), dim3(kSumThreads), stream, (const double*)a.partials,
                  tiles, per, a.partials + 2 * tiles, a.ticket, units * kUnitElems, acc3, accumulate);
  }
  if (tiles <= kDirectTiles)
    return launch(sums_final_kernel, dim3(1), dim3(kSumThreads), stream, (const double*)a.partials, tiles,
                  units * kUnitElems, acc3, accumulate);
  const int64_t per = (tiles + kMidGroups - 1) / kMidGroups;
  double* mid = a.partials + 2 * tiles;
  e = launch(sums_mid_kernel, dim3(kMidGroups), dim3(kThreads), stream, (const double*)a.partials,
             tiles, per, mid);
  if (e != hipSuccess) return e;
  return launch(sums_final_kernel, dim3(1), dim3(kSumThreads), stream, (const double*)mid,
                (int64_t)kMidGroups, units * kUnitElems, acc3, accumulate);
}

hipError_t launch_stats(int64_t n, const uint16_t* xt, const uint16_t* xr, const uint16_t* yt,
                        const uint16_t* yr, double* acc3, int accumulate, double* partials,
                        hipStream_t stream) {
  const int groups = (int)stats_groups(n);
  hipError_t e = launch(stats_partial_kernel, dim3(groups), dim3(kThreads), stream, xt, xr, yt, yr,
                        n, partials);
  if (e != hipSuccess) return e;
  return launch(sums_final_kernel, dim3(1), dim3(kSumThreads), stream, (const double*)partials,
                (int64_t)groups, n, acc3, accumulate);
}

}  // namespace tfp4

namespace tfp4 {
int64_t set_encode_batch(int64_t groups) { return g_encode_batch.exchange(groups); }
int64_t set_wait_limit(int64_t polls) { return g_wait_limit.exchange(polls); }

hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const DeviceSyms* syms = nullptr;
  if ((e = device_syms(dev, &syms)) != hipSuccess) return e;
  *out = syms->scratch;
  return hipSuccess;
}

hipError_t read_wait_failures(uint64_t* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const DeviceSyms* syms = nullptr;
  if ((e = device_syms(dev, &syms)) != hipSuccess) return e;
  unsigned long long v = 0;
  if ((e = hipMemcpy(&v, syms->fails, sizeof(v), hipMemcpyDeviceToHost)) != hipSuccess) return e;
  *out = (uint64_t)v;
  return hipSuccess;
}

// ---- row-offset groups: workspace [offs | tstart | table | tile maxima]

namespace {
// [offs | tstart | table | tile maxima (slots) | published S words | flag |
// tile descriptors]: the table and maxima hold the two-pass schedule's
// entries (tiles of kTileUnits), at least as many as the single pass's
// (kOPTableTile); the S words ([G][64], one copy per group), the flag and the
// descriptors (one int4 per kOPTableTile tile) serve the single pass, which
// takes up to kMergeGroups groups.
struct OffsLayout {
  int64_t entries, b_offs, b_tstart, b_table, b_tpart, b_sword, b_big, b_desc, total;
};
OffsLayout offs_layout(int64_t rows, int64_t cols, int64_t G) {
  OffsLayout L{};
  const int64_t units = rows * (cols / kUnitElems);
  L.entries = (units + kTileUnits - 1) / kTileUnits + G;
  auto up8 = [](int64_t b) { return (b + 7) / 8 * 8; };
  L.b_offs = 0;
  L.b_tstart = up8(8 * (G + 1));
  L.b_table = L.b_tstart + up8(4 * (G + 1));
  L.b_tpart = L.b_table + 8 * L.entries;
  L.b_sword = L.b_tpart + 4 * L.entries;            // contiguous with the maxima (one fill clears both)
  const bool single = G <= kMergeGroups;
  L.b_big = up8(L.b_sword + (single ? 4 * 64 * G : 0));
  // the single pass's tile descriptors (16 bytes per kOPTableTile tile)
  L.b_desc = (L.b_big + (single ? 8 : 0) + 15) / 16 * 16;
  L.total = L.b_desc + (single ? 16 * ((units + kOPTableTile - 1) / kOPTableTile + G) : 0);
  return L;
}

// Derives offs / tstart / table in the workspace; fills the map's fields.
hipError_t offs_prepare(int64_t rows, int64_t cols, int64_t G, const int64_t* off_in, float* gout,
                        void* work, TileMap* m, hipStream_t stream) {
  const OffsLayout L = offs_layout(rows, cols, G);
  uint8_t* w = static_cast<uint8_t*>(work);
  *m = TileMap{};
  m->offs = reinterpret_cast<const int64_t*>(w + L.b_offs);
  m->tstart = reinterpret_cast<const int32_t*>(w + L.b_tstart);
  m->table = reinterpret_cast<const int2*>(w + L.b_table);
  m->tpart = reinterpret_cast<const uint32_t*>(w + L.b_tpart);
  m->tu = kTileUnits;
  m->upr = cols / kUnitElems;
  m->groups = G;
  m->units = rows * m->upr;
  if (G <= kMergeGroups)
    return launch(offs_table_kernel, dim3((unsigned)max((L.entries + kThreads - 1) / kThreads, (int64_t)1)),
                  dim3(kThreads), stream, off_in, G, rows, m->upr, L.entries,
                  reinterpret_cast<int64_t*>(w + L.b_offs), reinterpret_cast<int32_t*>(w + L.b_tstart), gout,
                  reinterpret_cast<int2*>(w + L.b_table), (int64_t)kTileUnits, (int32_t*)nullptr, (int64_t)0,
                  (int4*)nullptr, (uint32_t*)nullptr, (int64_t)0);
  hipError_t e = launch(offs_prep_kernel, dim3(1), dim3(kThreads), stream, off_in, G, rows, m->upr,
                        reinterpret_cast<int64_t*>(w + L.b_offs), reinterpret_cast<int32_t*>(w + L.b_tstart),
                        gout);
  if (e != hipSuccess) return e;
  return launch(tile_table_kernel, dim3((unsigned)((L.entries + kThreads - 1) / kThreads)), dim3(kThreads),
                stream, m->tstart, G, L.entries, reinterpret_cast<int2*>(w + L.b_table));
}
}  // namespace

int64_t offs_work_bytes(int64_t rows, int64_t cols, int64_t groups) {
  return offs_layout(rows, cols, groups).total;
}

int64_t offs_entries(int64_t rows, int64_t cols, int64_t groups) {
  return offs_layout(rows, cols, groups).entries;
}

namespace {
// Single-pass encode of row-offset groups (onepass_encode_kernel over the
// device-built table of kOPTableTile-unit tiles) when the device holds the
// grid and the groups are few enough for their S words; *used tells whether
// it ran.
hipError_t launch_onepass_table(int bits, int64_t rows, int64_t cols, int64_t G, const int64_t* off_in,
                                const uint16_t* x, uint8_t* plane, uint8_t* scales, float* gout, uint16_t* y,
                                void* work, hipStream_t stream, bool* used) {
  *used = false;
  if (G > kMergeGroups) return hipSuccess;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipSuccess;
  const void* k = onepass_kernel(bits, y != nullptr, true);
  const int64_t cap = onepass_capacity(k, dev);
  if (cap < 2) return hipSuccess;
  const int64_t W = cap - 1;
  const OffsLayout L = offs_layout(rows, cols, G);
  const int64_t upr = cols / kUnitElems;
  const int64_t entries = (rows * upr + kOPTableTile - 1) / kOPTableTile + G;   // <= L.entries
  const int64_t rounds = ((entries + W - 1) / W + 1) & ~(int64_t)1;
  if (entries + 4 * W > INT32_MAX) return hipSuccess;
  const DeviceSyms* syms = nullptr;
  hipError_t e = device_syms(dev, &syms);
  if (e != hipSuccess) return e;
  uint8_t* w = static_cast<uint8_t*>(work);
  e = launch(offs_table_kernel, dim3((unsigned)max((entries + kThreads - 1) / kThreads, (int64_t)1)), dim3(kThreads),
             stream, off_in, G, rows, upr, entries, reinterpret_cast<int64_t*>(w + L.b_offs),
             reinterpret_cast<int32_t*>(w + L.b_tstart), gout, reinterpret_cast<int2*>(w + L.b_table),
             (int64_t)kOPTableTile, reinterpret_cast<int32_t*>(w + L.b_big), W + 1,
             reinterpret_cast<int4*>(w + L.b_desc), reinterpret_cast<uint32_t*>(w + L.b_tpart),
             L.entries + 64 * G);
  if (e != hipSuccess) return e;
  OnePassArgs a{};
  a.x = reinterpret_cast<const uint4*>(x);
  a.groups = (int)G;
  a.T = (int)W;
  a.Q = 1;
  a.L = kOPTableTile;
  a.rounds = (int)rounds;
  a.copies = 1;
  a.slots = reinterpret_cast<uint32_t*>(w + L.b_tpart);
  a.sword = reinterpret_cast<uint32_t*>(w + L.b_sword);
  a.gout = gout;
  a.plane = plane;
  a.scales = scales;
  a.y = reinterpret_cast<uint4*>(y);
  a.offs = reinterpret_cast<const int64_t*>(w + L.b_offs);
  a.tstart = reinterpret_cast<const int32_t*>(w + L.b_tstart);
  a.desc = reinterpret_cast<const int4*>(w + L.b_desc);
  a.big = reinterpret_cast<const int32_t*>(w + L.b_big);
  a.entries = (int)entries;
  a.upr = (int)upr;
  // (the prep kernel above cleared the slots and S words)
  e = onepass_enqueue(k, a, W + 1, a.slots, 0, dev, syms, stream);
  if (e == hipSuccess) *used = true;
  return e;
}
}  // namespace

hipError_t launch_encode_offsets(int bits, int64_t rows, int64_t cols, int64_t G, const int64_t* off_in,
                                 const uint16_t* x, uint8_t* plane, uint8_t* scales, float* gout,
                                 uint16_t* y, void* work, hipStream_t stream) {
  // One pass over the input (unless a batch size was set to force two passes)
  if (g_encode_batch.load(std::memory_order_relaxed) == 0) {
    bool used = false;
    const hipError_t e1 = launch_onepass_table(bits, rows, cols, G, off_in, x, plane, scales, gout, y, work, stream,
                                               &used);
    if (e1 != hipSuccess || used) return e1;
  }
  // Two passes: the tile maxima of every table entry, then quantize with each
  // group's S from its tiles' maxima.
  QuantArgs a{};
  hipError_t e = offs_prepare(rows, cols, G, off_in, gout, work, &a.map, stream);
  if (e != hipSuccess) return e;
  const int64_t entries = offs_layout(rows, cols, G).entries;
  a.x = reinterpret_cast<const uint4*>(x);
  a.gout = gout;
  a.plane = plane;
  a.scales = scales;
  a.y = reinterpret_cast<uint4*>(y);
  a.qblocks = entries;
  e = launch(tile_amax_kernel, dim3((unsigned)entries), dim3(kThreads), stream, a.map, a.x,
             const_cast<uint32_t*>(a.map.tpart));
  if (e != hipSuccess) return e;
  return quant_plane<0>(bits, y != nullptr, 3, false, a, entries, stream);
}

hipError_t launch_guided_offsets(int bits, int64_t rows, int64_t cols, int64_t G, const int64_t* off_in,
                                 const uint16_t* x, const uint8_t* guide, const uint8_t* scales,
                                 const float* gscale, uint16_t* y, uint8_t* codes, void* work,
                                 hipStream_t stream) {
  GuidedArgs a{};
  hipError_t e = offs_prepare(rows, cols, G, off_in, nullptr, work, &a.map, stream);
  if (e != hipSuccess) return e;
  const int64_t entries = offs_layout(rows, cols, G).entries;
  a.x = reinterpret_cast<const uint4*>(x);
  a.guide = guide;
  a.scales = scales;
  a.gscale = gscale;
  a.y = reinterpret_cast<uint4*>(y);
  a.codes = reinterpret_cast<uint32_t*>(codes);
  return guided_pack<0, 2>(bits, false, codes != nullptr, false, false, a, entries, stream);
}
}  // namespace tfp4
