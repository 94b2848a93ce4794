// MXFP4 quantize / pack on the GPU: rows of fp32 or bf16 weights -> E2M1 codes
// (two per byte, even element in the low nibble) and one E8M0 scale byte per
// 32-element block ([P3-FP4] 4-bit values sharing a per-block scale; [MX]
// conversion), the direction opposite to the layer's decode, for preparing
// expert weights on the device.
//
// Rule (one block of 32 values v): amax = max |v|; shared exponent
// X = floor(log2 amax) - 2 (E2M1's largest exponent is 2), clamped to
// [-127, 127], X = -127 when amax = 0; the scale byte is X + 127.  Each
// element goes to the E2M1 magnitude nearest |v| / 2^X, a tie to the one with
// an even mantissa bit, and above 6 to 6; the sign bit is set when v < 0.
//
// Layout of the work: a wave quantizes 16 blocks at a time, every load
// instruction reading 1 KiB of contiguous input (see k_quantize); a block's
// maximum comes from lane exchanges within its lane group.  The shared
// exponent is taken from the fp32 bit pattern of the maximum with integer
// operations.  The codes come from the hardware's scaled E2M1 convert, two
// per instruction, for every block whose X is at least -120; below that
// (blocks of values under 2^-118) they come from comparisons of the fp32 bit
// patterns with the decision points t 2^X (t = 0.25, 0.75, ..., 5: at most
// three significant bits, exact fp32 values built with shifts), which do not
// depend on how the hardware treats subnormal operands.  HBM-bound: 4.5 bytes
// per element (fp32 in) or 2.5 (bf16 in).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "moe_mxfp4.h"

namespace moe_q {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// fp32 bit pattern of m 2^p for a small odd integer m (1, 3, 5, 7) and
// -149 <= p, p + floor(log2 m) <= 127.
__device__ __forceinline__ uint32_t f32_bits_of(uint32_t m, int p) {
  const int n = 31 - __builtin_clz(m);  // floor(log2 m)
  const int ex = p + n + 127;
  if (ex >= 1) return ((uint32_t)ex << 23) | ((m << (23 - n)) & 0x7FFFFFu);
  return m << (p + 149);  // subnormal: m 2^p = (m 2^(p + 149)) 2^-149
}

// floor(log2 |v|) of a nonzero finite fp32 pattern without its sign bit.
__device__ __forceinline__ int ilog2_bits(uint32_t a) {
  const int ex = (int)(a >> 23);
  if (ex > 0) return ex - 127;
  return (31 - __builtin_clz(a)) - 149;  // subnormal
}

// Smallest shared exponent for which the hardware convert below is taken.
// From 2^-120 up, the scale 2^X is a normal fp32 value, and every element
// that can round to a nonzero code (|v| >= 2^(X-2) >= 2^-122) is normal too,
// so the convert sees exact operands; blocks below it take the bit-pattern
// comparisons.
constexpr int kHwMinX = -120;

// Two E2M1 codes of v0 / sc and v1 / sc (sc a power of two) into byte i of
// word (v0 in the low nibble); the byte index must be a literal.
__device__ __forceinline__ uint32_t cvt_pair_fp4(uint32_t word, float v0, float v1, float sc, int i) {
  switch (i) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v0, v1, sc, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v0, v1, sc, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v0, v1, sc, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v0, v1, sc, 3);
  }
}

// The codes of one block from its elements' patterns: every lane of the
// block's lane group holds N of them; the group (G lanes, aligned) exchanges
// its maximum.  Returns the lane's N codes packed (element 0 in the low
// nibble) and the block's X.
//
// Common case: gfx950's scaled convert (v_cvt_scalef32_pk_fp4_f32) turns two
// fp32 values into two E2M1 codes in one instruction.  It divides by the
// scale's power of two (exact here), rounds to the nearest E2M1 value with
// ties to the even mantissa bit, saturates at 6 and copies the sign bit, so
// it gives exactly the rule above except for a negative zero (sign bit set,
// where the rule sets it only for v < 0): a negative zero is passed as +0.
template <int N, int G>
__device__ __forceinline__ uint32_t block_codes(const uint32_t (&u)[N], int& Xout) {
  static_assert(N % 2 == 0 && N <= 8, "pairs of elements, one byte of codes each");
  uint32_t a[N];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    a[i] = u[i] & 0x7FFFFFFFu;
    amax = max(amax, a[i]);
  }
#pragma unroll
  for (int o = 1; o < G; o <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o));
  const int X = amax ? min(max(ilog2_bits(amax) - 2, -127), 127) : -127;
  Xout = X;
  uint32_t word = 0;
  if (X >= kHwMinX) {
    const float sc = __uint_as_float((uint32_t)(X + 127) << 23);
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float v0 = __uint_as_float(a[2 * i] ? u[2 * i] : 0u);
      const float v1 = __uint_as_float(a[2 * i + 1] ? u[2 * i + 1] : 0u);
      word = cvt_pair_fp4(word, v0, v1, sc, i);
    }
    return word;
  }
  // decision points t 2^X, t = 1/4, 3/4, 5/4, 7/4, 5/2, 7/2, 5; at a tie the
  // even mantissa bit wins: strictly above for 1/4, 5/4, 5/2, 5 and at or
  // above for 3/4, 7/4, 7/2
  const uint32_t d0 = f32_bits_of(1, X - 2), d1 = f32_bits_of(3, X - 2), d2 = f32_bits_of(5, X - 2),
                 d3 = f32_bits_of(7, X - 2), d4 = f32_bits_of(5, X - 1), d5 = f32_bits_of(7, X - 1),
                 d6 = f32_bits_of(5, X);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t code = (uint32_t)(a[i] > d0) + (uint32_t)(a[i] >= d1) + (uint32_t)(a[i] > d2) +
                          (uint32_t)(a[i] >= d3) + (uint32_t)(a[i] > d4) + (uint32_t)(a[i] >= d5) +
                          (uint32_t)(a[i] > d6);
    // sign bit for v < 0 (a negative zero keeps code 0 without it)
    word |= (code | ((u[i] >> 31) && a[i] ? 8u : 0u)) << (4 * i);
  }
  return word;
}

// A wave takes 16 blocks at a time, kU chunks of them per round with all
// the round's loads issued first (kU = 4 for fp32, 2 for bf16: the fastest
// measured on MI355X).  fp32: two 1 KiB loads per chunk, lane l holding
// elements 4l..4l+3 of each half (8 lanes per block); bf16: one 1 KiB load,
// lane l holding elements 8l..8l+7 (4 lanes per block).  Every load
// instruction reads 1 KiB of contiguous input; chunks past the end re-read
// the last chunk (in bounds) and store nothing.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) k_quantize(const void* w, int64_t nblocks, uint8_t* packed,
                                                       uint8_t* scales) {
  constexpr int kH = BF16 ? 1 : 2;  // 1 KiB loads per chunk
  constexpr int kU = BF16 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t nchunks = (nblocks + 15) / 16;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w);
  for (int64_t c0 = wave; c0 < nchunks; c0 += kU * nwaves) {
    u32x4_t r[kU][kH];
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int64_t c = min(c0 + q * nwaves, nchunks - 1);
#pragma unroll
      for (int hf = 0; hf < kH; ++hf) {
        // the last chunk may be partial: its lanes past the end read a clamped piece
        const int64_t piece = min(c * 64 * kH + hf * 64 + lane, nblocks * 4 * kH - 1);
        r[q][hf] = src[piece];
      }
    }
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int64_t c = c0 + q * nwaves;
      if (c >= nchunks) break;  // uniform
      if (BF16) {
        const int64_t b = c * 16 + (lane >> 2);
        uint32_t u[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t two = r[q][0][i];
          u[2 * i] = two << 16;
          u[2 * i + 1] = two & 0xFFFF0000u;
        }
        int X;
        const uint32_t word = block_codes<8, 4>(u, X);  // the block's four lanes agree on b < nblocks
        if (b < nblocks) {
          reinterpret_cast<uint32_t*>(packed)[c * 64 + lane] = word;
          if ((lane & 3) == 0) scales[b] = (uint8_t)(X + 127);
        }
      } else {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int64_t b = c * 16 + hf * 8 + (lane >> 3);
          uint32_t u[4] = {r[q][hf][0], r[q][hf][1], r[q][hf][2], r[q][hf][3]};
          int X;
          const uint32_t word = block_codes<4, 8>(u, X);
          if (b < nblocks) {
            reinterpret_cast<uint16_t*>(packed)[c * 128 + hf * 64 + lane] = (uint16_t)word;
            if ((lane & 7) == 0) scales[b] = (uint8_t)(X + 127);
          }
        }
      }
    }
  }
}

}  // namespace moe_q

extern "C" int moe_mxfp4_quantize(const void* w, int32_t dtype, int64_t rows, int64_t K, uint8_t* packed,
                                  uint8_t* scales, void* stream) {
  if (rows < 0 || K < 0 || (dtype != MOE_QDTYPE_F32 && dtype != MOE_QDTYPE_BF16)) return MOE_EINVAL;
  if (K % 32 != 0) return MOE_ESHAPE;
  const int64_t nblocks = rows * (K / 32);
  if (nblocks == 0) return MOE_OK;
  if (!w || !packed || !scales) return MOE_EINVAL;
  if ((uintptr_t)w % 16 || (uintptr_t)packed % 4) return MOE_EALIGN;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_EDEVICE;
  }
  // at most one chunk of 16 blocks per wave, and no more workgroups than the
  // CUs hold at once: every workgroup then runs from the start to the end,
  // with no second, partly filled wave of workgroups at the tail
  const void* kern = dtype == MOE_QDTYPE_BF16 ? (const void*)moe_q::k_quantize<true>
                                              : (const void*)moe_q::k_quantize<false>;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, moe_q::kThreads, 0) != hipSuccess ||
      per_cu < 1) {
    (void)hipGetLastError();
    return MOE_EDEVICE;
  }
  int64_t grid = ((nblocks + 15) / 16 + moe_q::kThreads / 64 - 1) / (moe_q::kThreads / 64);
  const int64_t cap = (int64_t)cus * per_cu;
  if (grid > cap) grid = cap;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MOE_QDTYPE_BF16)
    hipLaunchKernelGGL(moe_q::k_quantize<true>, dim3((unsigned)grid), dim3(moe_q::kThreads), 0, s, w, nblocks,
                       packed, scales);
  else
    hipLaunchKernelGGL(moe_q::k_quantize<false>, dim3((unsigned)grid), dim3(moe_q::kThreads), 0, s, w, nblocks,
                       packed, scales);
  if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
  return MOE_OK;
}

// ------------------------------------------------------------ host codec ---
// The same format on the host ([P3-FP4] 4-bit values plus one shared scale
// per small block; [MX] E2M1 elements, 32-element blocks, E8M0 scales), for
// callers that prepare or inspect expert weights in host memory.  Plain C++:
// the shared exponent comes from the fp32 bit pattern of the block maximum,
// the codes from a table of the rounding rule's decision points (the
// midpoints of neighbouring E2M1 magnitudes, which are exact in double).

namespace moe_q {

// floor(log2 a) for the bit pattern a (sign cleared) of a nonzero finite fp32.
static int host_ilog2(uint32_t a) {
  const int ex = (int)(a >> 23);
  if (ex > 0) return ex - 127;
  return (31 - __builtin_clz(a)) - 149;  // subnormal
}

static uint32_t host_bits(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  return u;
}

// E2M1 magnitude code (0..7) of q = |v| / 2^X >= 0: the nearest of 0, 0.5, 1,
// 1.5, 2, 3, 4, 6; at a midpoint the code with an even mantissa bit (even
// code), which is the lower neighbour at 0.25, 1.25, 2.5, 5 and the upper one
// at 0.75, 1.75, 3.5; above 6 the largest magnitude.
static uint32_t host_e2m1_code(double q) {
  if (q <= 0.25) return 0;
  if (q < 0.75) return 1;
  if (q <= 1.25) return 2;
  if (q < 1.75) return 3;
  if (q <= 2.5) return 4;
  if (q < 3.5) return 5;
  if (q <= 5.0) return 6;
  return 7;
}

// E2M1 code -> value: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
// exponent field 0 holds 0 and 0.5.
static float host_e2m1_value(uint32_t code) {
  static const float kMag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const float m = kMag[code & 7u];
  return (code & 8u) ? -m : m;
}

}  // namespace moe_q

extern "C" int moe_mxfp4_quantize_host(const float* w, int64_t rows, int64_t K, uint8_t* packed, uint8_t* scales) {
  using namespace moe_q;
  if (rows < 0 || K < 0) return MOE_EINVAL;
  if (K % 32) return MOE_ESHAPE;
  if (rows == 0 || K == 0) return MOE_OK;
  if (!w || !packed || !scales) return MOE_EINVAL;
  const int64_t n = rows * K;
  for (int64_t i = 0; i < n; ++i)
    if ((host_bits(w[i]) & 0x7F800000u) == 0x7F800000u) return MOE_EINVAL;  // inf or NaN
  const int64_t nb = K / 32;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* v = w + r * K + b * 32;
      uint32_t amax = 0;
      for (int i = 0; i < 32; ++i) {
        const uint32_t a = host_bits(v[i]) & 0x7FFFFFFFu;
        if (a > amax) amax = a;  // finite fp32 magnitudes order like their bit patterns
      }
      int X = amax == 0 ? -127 : host_ilog2(amax) - 2;
      if (X < -127) X = -127;
      if (X > 127) X = 127;
      scales[r * nb + b] = (uint8_t)(X + 127);
      uint8_t* out = packed + r * (K / 2) + b * 16;
      for (int i = 0; i < 32; i += 2) {
        uint32_t c[2];
        for (int h = 0; h < 2; ++h) {
          const float x = v[i + h];
          const double q = ldexp(fabs((double)x), -X);  // exact: a power-of-two scaling of an fp32 value
          c[h] = host_e2m1_code(q) | ((host_bits(x) >> 31) && x != 0.0f ? 8u : 0u);
        }
        out[i / 2] = (uint8_t)(c[0] | (c[1] << 4));
      }
    }
  }
  return MOE_OK;
}

extern "C" int moe_mxfp4_dequantize_host(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t K,
                                         float* w) {
  using namespace moe_q;
  if (rows < 0 || K < 0) return MOE_EINVAL;
  if (K % 32) return MOE_ESHAPE;
  if (rows == 0 || K == 0) return MOE_OK;
  if (!packed || !scales || !w) return MOE_EINVAL;
  const int64_t nb = K / 32;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint32_t s = scales[r * nb + b];
      // 2^(s-127) in double (exact for every byte), NaN for 255
      const double sc = s == 255u ? (double)NAN : ldexp(1.0, (int)s - 127);
      const uint8_t* in = packed + r * (K / 2) + b * 16;
      float* o = w + r * K + b * 32;
      for (int i = 0; i < 16; ++i) {
        o[2 * i] = (float)((double)host_e2m1_value(in[i] & 0xFu) * sc);
        o[2 * i + 1] = (float)((double)host_e2m1_value(in[i] >> 4) * sc);
      }
    }
  }
  return MOE_OK;
}
