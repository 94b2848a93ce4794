// Device-side building blocks for the MXFP4 MoE layer on gfx950 (CDNA4, wave64).
//
// MXFP4 ([MX]: OCP Microscaling v1.0, the format the "MiMo x TileRT" pages name
// for the experts): E2M1 codes, two per byte (even element in the low nibble),
// one E8M0 scale byte per 32 elements.  Decoding uses gfx950's scaled FP4
// converts, which turn one byte (two codes) into two bf16 or two fp32 values
// multiplied by the block scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// E8M0 byte s -> the fp32 scale operand of the scaled converts below: s in
// the exponent field.  As an fp32 value this is 2^(s-127) for s in [1, 254]
// and +0 for s = 0, but the converts use only the operand's exponent field,
// so s = 0 also decodes as 2^-127 (the format's value), subnormal results
// included (measured on MI355X for every code at s = 0, 1, 2; the GPU tests
// check blocks of bytes 0, 1 and 254 against the oracle).  s = 255 (NaN in the
// format) is +inf here and not supported.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __builtin_bit_cast(float, s << 23);
}

// Byte `sel` (0..3) of `w` -> two bf16 (low nibble in .x), times `scale`.
template <int SEL>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16x2(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL);
}

// Byte `sel` (0..3) of `w` -> two fp32 (low nibble in .x), times `scale`.
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
}

// acc + a.x*b.x + a.y*b.y (bf16 products, fp32 accumulation).
__device__ __forceinline__ float dot2_bf16(bf16x2_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// 32 packed codes (one 16-byte load, one block) against 32 bf16 activations
// held as four 16-byte pieces (piece q = elements 8q..8q+7).
__device__ __forceinline__ float dot32_bf16(const u32x4_t w, float scale, const u32x4_t* xq, float acc) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4_t xv = xq[q];
    acc = dot2_bf16(fp4x2_to_bf16x2<0>(ws[q], scale), xv.x, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<1>(ws[q], scale), xv.y, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<2>(ws[q], scale), xv.z, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<3>(ws[q], scale), xv.w, acc);
  }
  return acc;
}

// 32 packed codes (one 16-byte chunk) -> 16 bf16 pairs times the block scale
// (pair i = elements 2i, 2i+1), for reuse against several tokens.
__device__ __forceinline__ void decode32_bf16(const u32x4_t w, float scale, bf16x2_t (&v)[16]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[4 * q + 0] = fp4x2_to_bf16x2<0>(ws[q], scale);
    v[4 * q + 1] = fp4x2_to_bf16x2<1>(ws[q], scale);
    v[4 * q + 2] = fp4x2_to_bf16x2<2>(ws[q], scale);
    v[4 * q + 3] = fp4x2_to_bf16x2<3>(ws[q], scale);
  }
}

// acc + the 16 decoded pairs against 32 bf16 activations held as four 16-byte
// pieces, in the same order as dot32_bf16 (so the sums are identical).
__device__ __forceinline__ float dot32_bf16_dec(const bf16x2_t (&v)[16], const u32x4_t* xq, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4_t xv = xq[q];
    acc = dot2_bf16(v[4 * q + 0], xv.x, acc);
    acc = dot2_bf16(v[4 * q + 1], xv.y, acc);
    acc = dot2_bf16(v[4 * q + 2], xv.z, acc);
    acc = dot2_bf16(v[4 * q + 3], xv.w, acc);
  }
  return acc;
}

// ---- MFMA operands (v_mfma_f32_16x16x32_bf16, wave64) ----
// A (16 x 32): lane l holds row l % 16, K elements 8(l / 16) .. +8.
// B (32 x 16): lane l holds column l % 16, K elements 8(l / 16) .. +8.
// D (16 x 16, fp32): lane l holds column l % 16, rows 4(l / 16) .. +4.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// D = A B + C on 16x16 fp32 tiles, K = 4 per instruction, fp32 products and
// sums: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and holds
// D[4 (l / 16) + r][l % 16] in element r.
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One 16-byte chunk (32 codes, one scale block) -> four A operands: operand s
// holds elements 8s .. 8s+7 of the chunk, times the block scale (exact).
__device__ __forceinline__ void decode_chunk_a(const u32x4_t w, float scale, bf16x8_t (&a)[4]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x2_t p0 = fp4x2_to_bf16x2<0>(ws[s], scale), p1 = fp4x2_to_bf16x2<1>(ws[s], scale);
    const bf16x2_t p2 = fp4x2_to_bf16x2<2>(ws[s], scale), p3 = fp4x2_to_bf16x2<3>(ws[s], scale);
    a[s] = bf16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  }
}

// fp32 -> bf16 hi + bf16 lo with hi + lo = v to 16 significant bits (RNE both).
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = (__bf16)v;
  lo = (__bf16)(v - (float)hi);
}

// 32 packed codes (one 16-byte chunk) -> 32 fp32 values times the block scale.
__device__ __forceinline__ void decode32_f32(const u32x4_t w, float scale, float (&v)[32]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x2_t a;
    a = fp4x2_to_f32x2<0>(ws[q], scale);
    v[8 * q + 0] = a.x;
    v[8 * q + 1] = a.y;
    a = fp4x2_to_f32x2<1>(ws[q], scale);
    v[8 * q + 2] = a.x;
    v[8 * q + 3] = a.y;
    a = fp4x2_to_f32x2<2>(ws[q], scale);
    v[8 * q + 4] = a.x;
    v[8 * q + 5] = a.y;
    a = fp4x2_to_f32x2<3>(ws[q], scale);
    v[8 * q + 6] = a.x;
    v[8 * q + 7] = a.y;
  }
}

// acc + sum_i v[i] * h[i] over 32 values, fp32 FMA in index order.
__device__ __forceinline__ float dot32(const float (&v)[32], const float* h, float acc) {
#pragma unroll
  for (int i = 0; i < 32; ++i) acc = fmaf(v[i], h[i], acc);
  return acc;
}

// 16-byte streaming load of weight bytes that are read exactly once per call.
__device__ __forceinline__ u32x4_t ld_stream16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Bits -> float through a by-value parameter.  (Do not write
// __builtin_bit_cast(float, v.z) on an ext_vector element: this toolchain
// lowers it as a read of element 0.)
__device__ __forceinline__ float u2f(uint32_t v) { return __builtin_bit_cast(float, v); }

// Value known to be equal in all lanes of the wave, moved to a scalar register.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// bf16 bits -> fp32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// gfx950 lane swaps across rows.  With the same register as both operands,
// permlane16_swap returns {row 2n, row 2n+1} and permlane32_swap returns
// {lanes 0-31, lanes 32-63}, each in both lanes of a pair: element 0 holds
// the lower lane's value, element 1 the upper lane's (partner = lane ^ 16,
// lane ^ 32).  No LDS round trip, unlike a bpermute shuffle.
__device__ __forceinline__ void swap16(uint32_t v, uint32_t& lo, uint32_t& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  lo = r[0];
  hi = r[1];
}
__device__ __forceinline__ void swap32(uint32_t v, uint32_t& lo, uint32_t& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  lo = r[0];
  hi = r[1];
}

// Sum over the 64 lanes of a wave; every lane receives the same total (the
// operands of each step are added in lane order, so all lanes agree bit for
// bit).  Row steps: DPP xor 1, xor 2, half-row mirror, row mirror; then the
// two cross-row swaps.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  uint32_t a, b;
  swap16(__builtin_bit_cast(uint32_t, v), a, b);
  v = u2f(a) + u2f(b);
  swap32(__builtin_bit_cast(uint32_t, v), a, b);
  return u2f(a) + u2f(b);
}

// Maximum of an unsigned 32-bit value over the 64 lanes; every lane gets it.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u<0x140>(v));  // row_mirror
  uint32_t a, b;
  swap16(v, a, b);
  v = max(a, b);
  swap32(v, a, b);
  return max(a, b);
}

// Maximum of a 64-bit key over the 64 lanes; every lane receives it.
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  // high words first, then the low words of the lanes holding the top high
  // word (a key with a zero low word never wins a tie, which callers avoid)
  const uint32_t hi = wave_max_u32((uint32_t)(k >> 32));
  const uint32_t lo = wave_max_u32((uint32_t)(k >> 32) == hi ? (uint32_t)k : 0u);
  return ((uint64_t)hi << 32) | lo;
}

// Eight per-lane partial sums v[0..7] -> every lane receives the wave-wide
// total of value (lane >> 3).  Reduce-scatter: exchange half of the values
// across lane bits 5, 4 and 3, then sum the remaining value over lane bits
// 0..2.  Costs ~30 VALU ops and 6 lane swaps instead of 8 full reductions.
__device__ __forceinline__ float reduce8(const float v[8]) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
  float w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float keep = b5 ? v[i + 4] : v[i];
    const float send = b5 ? v[i] : v[i + 4];
    uint32_t lo, hi;
    swap32(__builtin_bit_cast(uint32_t, send), lo, hi);
    w[i] = keep + u2f(b5 ? lo : hi);  // the partner lane's `send`
  }
  float x[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = b4 ? w[i + 2] : w[i];
    const float send = b4 ? w[i] : w[i + 2];
    uint32_t lo, hi;
    swap16(__builtin_bit_cast(uint32_t, send), lo, hi);
    x[i] = keep + u2f(b4 ? lo : hi);
  }
  float y;
  {
    const float keep = b3 ? x[1] : x[0];
    const float send = b3 ? x[0] : x[1];
    y = keep + dpp_f<0x128>(send);  // row_ror:8 = lane ^ 8 within a row of 16
  }
  y += dpp_f<0xB1>(y);   // xor 1
  y += dpp_f<0x4E>(y);   // xor 2
  y += dpp_f<0x141>(y);  // half-row mirror: the other quad of the 8
  return y;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Inclusive prefix sum over the lanes of a wave.
// Row shifts (row_shr:1,2,4,8; lanes without a source add 0) scan each row of
// 16, then row_bcast:15 and row_bcast:31 carry the row totals down the wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31 into rows 2, 3
  return v;
}

// ---------------------------------------------------------------- atomics ---
__device__ __forceinline__ uint32_t ld_acquire(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_acq_rel(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_release(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Epoch-tagged 32-bit values: {value, tag} in one 64-bit word, written and
// read with single-copy-atomic agent-scope accesses (coherent across the
// chip's L2 slices without cache flushes).  A consumer accepts a word only if
// its tag equals the current call's tag, so no barrier or fence is needed
// between producer and consumer, and stale words of earlier calls never pass.
__device__ __forceinline__ void st_tagged(uint64_t* p, uint32_t bits, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_ok(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

// Buffer descriptor over `bytes` bytes at `base` (a wave-uniform address);
// reads past the end return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Two tagged words {v0, tag, v1, tag} with one 16-byte store that writes
// through the L2 (sc1, the cache policy of st_tagged's 8-byte atomic stores).
// An aligned 16-byte store reaches memory in one piece, so readers (16-byte
// coherent loads, each 8-byte half read whole) never see half a word; the
// stores of neighbouring lanes then fill whole 128-byte lines instead of
// 8-byte pieces of them.
__device__ __forceinline__ void st_tagged2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint32_t v0, uint32_t v1,
                                           uint32_t tag) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v0, tag, v1, tag}, r, byte_off, 0, 16);
}

// 16-byte agent-coherent load (sc1: not served from a stale L2 line of
// another call) of two tagged words {lo value, lo tag, hi value, hi tag}.
// Each aligned 8-byte half is read single-copy atomically.  Unlike atomic
// loads, several of these stay in flight at once.
__device__ __forceinline__ u32x4_t ld_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16);
}
// The same through this XCD's L2 (no cache-policy bits): several times
// faster under full load, but the L2 may hold the line from an earlier call
// (the words then carry an old tag).  Used for first attempts after
// invalidate_l2; a word whose tag matches is exact either way, since each
// tagged word is written once per call.
__device__ __forceinline__ u32x4_t ld_cached16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// 16-byte streaming load (nt: read once) and byte load through a buffer
// descriptor, at a 32-bit byte offset.
__device__ __forceinline__ u32x4_t ld_stream16_buf(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2);
}
__device__ __forceinline__ uint32_t ld_byte_buf(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, byte_off, 0, 0);
}
// 8-byte load through a buffer descriptor and the L2 (byte_off a multiple of 8).
__device__ __forceinline__ u32x2_t ld_cached8_buf(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
}

// Drops this XCD's L2 lines (and the CU's vector cache), so that later cached
// reads of the workspace fetch what the other XCDs wrote through to memory.
// Issued without a wait: later waits of the wave cover it.
__device__ __forceinline__ void invalidate_l2() { __asm__ __volatile__("buffer_inv sc1" ::: "memory"); }

__device__ __forceinline__ float tag_f32(uint64_t w) { return __builtin_bit_cast(float, (uint32_t)w); }
__device__ __forceinline__ int tag_i32(uint64_t w) { return (int)(uint32_t)w; }

}  // namespace moe
