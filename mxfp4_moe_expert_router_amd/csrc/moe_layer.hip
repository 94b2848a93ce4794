// MXFP4 MoE expert layer for AMD Instinct MI355X (gfx950): kernels and C ABI.
//
// The layer (router -> top-k -> permutation -> MXFP4 gate/up + SwiGLU -> MXFP4
// down -> gate-weighted combine) follows the pages on the MiMo x TileRT system:
//  [P1-FP4] "MiMo x TileRT" (blog.hypho.cn), section "第一层：FP4 选择性量化":
//           experts in OCP MXFP4, router at higher precision;
//  [P1-BG]  same article, section "万亿参数推理为什么特别难": a token activates a
//           few experts; decode is bounded by bytes read per token;
//  [P3-FP4] "MiMo 把 1T 模型推到每秒千 token——FP4、DFlash 與常駐 kernel 的三層
//           co-design" (vatt-ghern.pages.dev), section "FP4：只量化 MoE expert，
//           其餘維持原精度": 4-bit blocks sharing one scale; precision-sensitive top-k;
//  [P3-PK]  same page, section "persistent engine kernel 與 warp specialization":
//           the pipeline as one resident kernel, no launch per operator;
//  [P5-FP4] "tech-implementation-2026-06-09" (shengyayun.com), section "关键实现细节
//           / 1.": expert gate_proj / up_proj / down_proj are the MXFP4 linears;
//  [P5-TRT] same page, section "3. TileRT 的"持久化内核"到底做了什么": MoE gate then
//           expert compute inside one resident kernel.
//
// Execution model.  The whole layer is ONE launch whose grid is one
// 512-thread workgroup per CU (all co-resident).  Steps hand data to each
// other through epoch-tagged words: a 64-bit {value, tag} written and read
// with single-copy-atomic, agent-coherent accesses.  A consumer spins (with a
// wall-clock watchdog) until the words it needs carry the current call's tag.
// There are no grid barriers, no cache-flushing fences and no read-modify-
// write atomics on the path: on MI355X one grid barrier over 256 workgroups
// costs tens of microseconds because device-scope atomics to one address
// serialize, while a tagged word costs one coherent store.  Deadlock freedom:
// every workgroup runs the steps in the same order and a step only waits on
// words produced by earlier steps of (possibly other) co-resident workgroups.
//
// Steps:
//   router   units (expert, 8 tokens), one workgroup each, its waves splitting d
//            -> tagged logits
//   top-k    one wave per token -> tagged {expert id, gate} records, 8 copies
//   permute  every workgroup builds the (expert, token) permutation in LDS
//   gate/up  small batches: all of x resident in LDS, each wave streams a
//            contiguous range of (expert, row) pairs of W_gate/W_up;
//            large batches: workgroup units with x staged per token group
//            -> tagged h = silu(W_gate x) * (W_up x)
//   down     each wave streams a contiguous range of (expert, row) of W_down,
//            8 rows per step, h of the expert's tokens held in registers
//            -> tagged gate * y in the token's slot
//   combine  out[t] = sum of the token's k slots, in slot order
//
// Hot loops: a lane owns 16-byte chunks (32 codes = one scale block) of a row,
// so a wave-wide load reads 1 KiB contiguous; the next rows' loads are issued
// before the current rows are computed.  gate/up decode codes to bf16 with the
// block scale folded in (v_cvt_scalef32_pk_bf16_fp4) and use bf16 dot2 with
// fp32 accumulation (x is bf16 and every E2M1 * 2^k is exact in bf16); down
// decodes to fp32 (v_cvt_scalef32_pk_f32_fp4) and uses fp32 FMA so h is never
// rounded.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "moe_device.h"
#include "moe_mxfp4.h"

namespace moe {

constexpr int kWG = 512;               // threads per workgroup
constexpr int kWaves = kWG / kWave;    // waves per workgroup
constexpr int kLdsMax = 160 * 1024 - 1024;  // dynamic LDS per workgroup (gfx950 has 160 KiB; static LDS needs a few bytes)
constexpr int kRouterTok = 8;          // tokens per router unit
constexpr int kRouterF4 = 4;           // float4 per lane of a router unit's wave (d / 8 <= 1024 columns)
constexpr int kRouterTileBytes = 8 * 16 * 16 * 4;  // router_mfma: one 16 x 16 fp32 tile per wave
constexpr int kRouterMfmaT = 64;       // router_mfma above this many tokens (router_step up to it)
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;
constexpr int kMaxD = 8192;
constexpr int kMaxF = 4096;
constexpr int kGUChunks = 4;           // 16-byte chunks per lane of a d-row (d <= 8192)
// Tokens per pass over a decoded gate/up row pair: 2 with x of every token in
// LDS (experts of the 1-8 token blocks mostly have one or two tokens; on
// MI355X 2 instead of 4 took the 8-token verify block from 248.6 to 246.0 us,
// the 4-token one from 140.5 to 134.9 and decode from 54.7 to 53.4, while the
// shared-routing 8-token block, with up to 7 tokens per expert, went from
// 185.4 to 188.0), 4 with x of the workgroup's own pairs (16-32 tokens).
template <bool XP>
constexpr int kGUTok = XP ? 4 : 2;
constexpr int kDnRows = 8;             // W_down rows per down step (at most; reduce8 width)
constexpr int kMaxGrid = 2048;
constexpr int kMaxLayers = 4096;        // layers of one stack call
constexpr int kMaxMaskWords = 4096;    // E * ceil(T/64)
constexpr int kTraceSlots = 16;        // wall-clock stamps per workgroup (trace option)
constexpr int kTopkRep = 8;            // copies of the top-k results (each read by 1/8 of the grid)
constexpr int kRounds = 8;             // work rounds of the small-batch gate/up step (see set_ranges)
// MFMA expert path (x does not fit in LDS)
constexpr int kKB = 128;               // K elements per block
constexpr int kDnTiles = 4;            // W_down tiles (16 rows) per wave
constexpr int kGUPass = 32;            // tokens per gate/up pass (2 groups of 16)
constexpr int kDnPass = 32;            // tokens per down pass (2 groups of 16)
constexpr int kTileRow = 272;          // LDS bytes per token row of an activation tile (256 + 16 pad)
constexpr int kGUK = 4;                // gate/up K blocks per step (8 KiB of codes per wave)
constexpr int kDnK = 2;                // down K blocks per step (8 KiB of codes per wave: whole 128-byte lines)
constexpr int kGUUnitRows = kWaves * 16;             // 128 row pairs
constexpr int kDnUnitRows = kWaves * kDnTiles * 16;  // 512 rows
constexpr size_t kMfmaLds = 2 * (size_t)kGUK * kGUPass * kTileRow;  // two activation tiles of a step

// Header words (first kHdrBytes of the workspace).
enum { kEpoch = 0, kStatus = 1, kAbort = 2, kWhere = 3, kWhat = 4, kStarted = 64 };
constexpr size_t kHdrBytes = (size_t)(kStarted + kMaxGrid) * 4;

struct Params {
  int T, d, F, E, k;
  const uint16_t* x;
  const float* wr;
  const uint8_t* packed;
  const uint8_t* scales;
  float* out;
  uint32_t* hdr;
  uint64_t* lgp;   // [T][E rounded up to even] tagged logits (two such arrays of partial sums, see router_halves)
  uint64_t* tk;    // [kTopkRep][T*k][2] tagged {expert id, gate} per slot, replicated
  uint64_t* hq;    // [T*k][F] tagged h, pair order
  uint64_t* yq;    // [T*k][d] tagged gate * y, slot order
  float* logits;   // plain copies for inspection
  int32_t* topk_idx;
  float* topk_w;
  int32_t* offsets;
  int32_t* sorted_slot;
  int32_t* pos;
  int32_t* active;
  int32_t* n_active;
  uint64_t* trace;    // [grid][kTraceSlots] wall-clock stamps, or null
  uint64_t spin_ticks;
  uint32_t withhold;  // test knob: top-k waits for a tag the router never writes
  uint32_t withhold_h;  // test knob: the down step waits for a tag gate/up never writes
  int mfma;           // 1: x does not fit in LDS, expert steps on MFMA
  int xmode;          // small-batch path: 0 x of every token in LDS, 1 x of the workgroup's pairs (see stage_pairs)
  int xrows;          // small-batch path: rows of x the LDS holds
  int narrow;         // 1: every byte offset into hq and yq fits in 32 bits (16-byte tagged stores)
  // A stack of layers on one residual stream r (r_0 = x0, x_l =
  // bf16(rmsnorm(r_l)), r_{l+1} = r_l + layer_l(x_l), out = r_L): the combine
  // adds the layer's output to r, which out holds.
  int stack_layers;   // L of the stack; 0: a lone layer (out = layer(x))
  int layer0;         // stack index of the launch's first layer
  const float* rin;   // stack: r_l of the layer (layer 0 reads x0 instead)
  float* rout;        // stack: where the layer writes r_{l+1}
  float* rbuf;        // stack: fp32 [T][d] workspace buffer; the one-launch stack
                      // alternates r between it and out (see k_stack)
  int nlayers;        // layers this launch runs (k_stack), 1 otherwise
  const uint16_t* x0; // the stack's input, bf16 [T][d] (r_0)
  uint16_t* xb;       // bf16 [T][d]: a layer's normalised input (the last one's after a call)
  size_t wr_stride;   // floats between layers' router weights
  size_t pk_stride;   // bytes between layers' packed experts
  size_t sc_stride;   // bytes between layers' scales
};

// ------------------------------------------------------------ LDS layout ----
// Shared by host (size) and device (carving).
struct LdsPlan {
  size_t xs, mask, tki, tkw, off, slot, act, cgu, cdn, misc, rt, total;
};

__host__ __device__ inline size_t al16(size_t v) { return (v + 15) & ~(size_t)15; }

// xrows > 0: the small-batch path with that many rows of x in LDS; 0: the
// MFMA path.
__host__ __device__ inline LdsPlan lds_plan(int T, int d, int E, int k, int xrows) {
  LdsPlan L;
  const size_t TK = (size_t)T * k;
  const size_t W = ((size_t)T + 63) / 64;
  const size_t mask_bytes = (size_t)E * W * 8;
  size_t o = 0;
  if (xrows > 0) {
    // rows of x stay resident; the permutation masks get their own space
    L.xs = o; o = al16(o + (size_t)xrows * d * 2);
    L.mask = o; o = al16(o + mask_bytes);
  } else {
    // the activation tiles of the MFMA path are used after the permutation is
    // built: the masks alias them
    size_t xs_bytes = kMfmaLds;
    if (mask_bytes > xs_bytes) xs_bytes = mask_bytes;
    L.xs = o; L.mask = o; o = al16(o + xs_bytes);
  }
  L.tki = o; o = al16(o + TK * 4);
  L.tkw = o; o = al16(o + TK * 4);
  L.off = o; o = al16(o + ((size_t)E + 1) * 4);
  L.slot = o; o = al16(o + TK * 4);
  L.act = o; o = al16(o + (size_t)E * 4);
  L.cgu = o; o = al16(o + ((size_t)E + 1) * 4);
  L.cdn = o; o = al16(o + ((size_t)E + 1) * 4);
  L.misc = o; o = al16(o + 64 * 4);
  L.rt = o; o = al16(o + (T > kRouterMfmaT ? kRouterTileBytes : 0));  // router_mfma's partial tiles
  L.total = o;
  return L;
}

struct Smem {
  u32x4_t* xs;
  uint64_t* mask;
  int* tki;
  float* tkw;
  int* off;
  int* slot;
  int* act;
  int* cgu;   // [n_active + 1] cumulative gate/up work per row, over active experts
  int* cdn;   // [n_active + 1] same for down
  float* rt;  // router_mfma's partial tiles (more than kRouterMfmaT tokens)
  int* misc;  // [0] n_active, [1] / [2] work counters, [8..8+kWaves) scan scratch, [16..50) round tables,
              // [50] / [51] staged x rows (xmode 1), [52] MFMA unit stride
};

// Round table of the small-batch expert steps (phase 0 gate/up, 1 down) in
// S.misc: kRounds chunk starts, then kRounds + 1 cumulative chunk lengths.
constexpr int kRoundTab = 2 * kRounds + 1;
constexpr int kMiscXBase = 50, kMiscXRows = 51;  // x rows staged in LDS (xmode 1): first pair, count
constexpr int kMiscStride = 52;                  // MFMA path: stride between a workgroup's units
__device__ __forceinline__ int* round_tab(const Smem& S, int phase) { return S.misc + 16 + phase * kRoundTab; }

__device__ __forceinline__ Smem carve(char* base, const Params& P, bool small) {
  const LdsPlan L = lds_plan(P.T, P.d, P.E, P.k, small ? P.xrows : 0);
  Smem S;
  S.xs = reinterpret_cast<u32x4_t*>(base + L.xs);
  S.mask = reinterpret_cast<uint64_t*>(base + L.mask);
  S.tki = reinterpret_cast<int*>(base + L.tki);
  S.tkw = reinterpret_cast<float*>(base + L.tkw);
  S.off = reinterpret_cast<int*>(base + L.off);
  S.slot = reinterpret_cast<int*>(base + L.slot);
  S.act = reinterpret_cast<int*>(base + L.act);
  S.cgu = reinterpret_cast<int*>(base + L.cgu);
  S.cdn = reinterpret_cast<int*>(base + L.cdn);
  S.misc = reinterpret_cast<int*>(base + L.misc);
  S.rt = reinterpret_cast<float*>(base + L.rt);
  return S;
}

// ------------------------------------------------------------ watchdog ------

__device__ __forceinline__ bool aborted(const Params& P, uint32_t tag) {
  return ld_relaxed(&P.hdr[kAbort]) == tag;
}

// Wait sites, recorded with the index waited on when a watchdog fires.
enum { kSiteLogits = 1, kSiteTopk = 2, kSiteH = 3, kSiteY = 4, kSiteStarted = 5, kSiteLayer = 6 };

__device__ __forceinline__ void raise_timeout(const Params& P, uint32_t tag, uint32_t site, uint32_t what) {
  st_relaxed(&P.hdr[kWhere], site);
  st_relaxed(&P.hdr[kWhat], what);
  st_relaxed(&P.hdr[kStatus], (uint32_t)MOE_ETIMEOUT);
  st_relaxed(&P.hdr[kAbort], tag);
}

// One spin round of a wave-level wait: true to retry, false to give up.
// Rounds back off exponentially from about 0.2 us up to 2^max_shift times
// that, so that waiting waves do not flood the memory system that the waves
// they wait for are using, without oversleeping much past the arrival.  The
// compiler memory barrier makes the caller's polling loads (plain buffer
// loads, not atomics) be issued again on the next round instead of being
// reused from registers.
__device__ __forceinline__ bool keep_waiting(const Params& P, uint32_t tag, uint64_t t0, uint32_t site,
                                             uint32_t what, int& round, int max_shift) {
  // the abort word (another wait timed out) is a round trip to memory: look
  // at it every 8th round only
  if ((round & 7) == 7 && aborted(P, tag)) return false;
  if (wall_clock64() - t0 > P.spin_ticks) {
    raise_timeout(P, tag, site, what);
    return false;
  }
  const int units = 1 << min(round, max_shift);
  for (int i = 0; i < units; ++i) __builtin_amdgcn_s_sleep(8);
  ++round;
  __asm__ __volatile__("" ::: "memory");
  return true;
}

// Tag of this call: epoch + 1, never 0 (a zero-filled workspace has tag 0).
// A launch that runs `nl` layers uses tags epoch + 1 .. epoch + nl, one per
// layer; they restart from 1 rather than reach 0xFFFFFFFF.
__device__ __forceinline__ uint32_t start_call(const Params& P, int wg, bool mark_started, int nl = 1) {
  __shared__ uint32_t s_tag;
  if (threadIdx.x == 0) {
    uint32_t e = ld_relaxed(&P.hdr[kEpoch]);
    if (e > 0xFFFFFFFEu - (uint32_t)nl) e = 0u;
    s_tag = e + 1u;
    if (mark_started) st_relaxed(&P.hdr[kStarted + wg], e + 1u);
  }
  __syncthreads();
  return s_tag;
}

__device__ __forceinline__ uint32_t next_epoch(uint32_t tag) { return tag >= 0xFFFFFFFEu ? 0u : tag; }

// Workgroup 0 closes the call: once every workgroup has read the epoch, the
// epoch advances so that the next call's tag differs from every word written
// by this one.
__device__ __forceinline__ void end_call(const Params& P, uint32_t tag, int G) {
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x < kWave) {
    const uint64_t t0 = wall_clock64();
  int round = 0;
    for (;;) {
      bool ok = true;
      for (int w = lane; w < G; w += kWave) ok &= (ld_relaxed(&P.hdr[kStarted + w]) == tag);
      if (__all(ok)) break;
      if (wall_clock64() - t0 > P.spin_ticks) {
        if (lane == 0) raise_timeout(P, tag, kSiteStarted, 0);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0) st_relaxed(&P.hdr[kEpoch], next_epoch(tag));
  }
}

// Trace option: the first wave of workgroup `wg` stamps the end of step `i`.
__device__ __forceinline__ void stamp(const Params& P, int wg, int i) {
  if (P.trace != nullptr && threadIdx.x == 0) P.trace[(size_t)wg * kTraceSlots + i] = wall_clock64();
}
// Trace option: waves 1..7 of workgroup `wg` stamp the end of their gate/up rows.
__device__ __forceinline__ void stamp_gu_wave(const Params& P, int wg) {
  const int wave = threadIdx.x / kWave;
  if (P.trace != nullptr && wave > 0 && (threadIdx.x & (kWave - 1)) == 0)
    P.trace[(size_t)wg * kTraceSlots + 8 + wave] = wall_clock64();
}

// ---------------------------------------------------------------- router ----
// logits[t][e] = sum_c x[t][c] * W_r[e][c] in fp32 ([P1-FP4]/[P3-FP4]: the
// router stays at higher precision than the experts).  Unit = (expert, group
// of 8 tokens), one workgroup: wave v covers columns [v*d/8, (v+1)*d/8) of
// the expert's row held in registers, the 8 per-wave partial sums of a logit
// are added in wave order.  XLDS: x comes from the LDS copy (piece-transposed,
// see stage_x), else from global memory.  `pre` (all threads) runs once, after
// the first unit's weight loads are issued: it overlaps the x staging with
// them.  All threads of the workgroup.
// Router for more than kRouterMfmaT tokens ([P1-FP4] higher-precision
// router): logits = x W_r^T in fp32 on v_mfma_f32_16x16x4_f32, so that W_r
// and x are read once per 16 x 16 tile instead of once per (expert, 8 tokens)
// (T=512: 58 us instead of 200).  A unit moves ~0.7 MB at one CU's share of
// the bandwidth (~30 us), so for fewer tokens, with fewer units than CUs,
// router_step's finer units finish first.  Unit =
// (16 experts, 16 or 32 tokens, all or half of the K blocks), one workgroup
// (router_token_blocks, router_halves); wave w sums the w-th eighth of the
// unit's K blocks of 16.  In K block j, lane l loads 4 consecutive K
// (16j + 4 (l / 16) .. +3) of expert row l % 16 and of token row l % 16, and
// MFMA step s uses element s of both (each step sums a permuted but matching
// set of 4 K).  The 8 partial tiles are added in wave order; a lane past the
// last expert or token reads a clamped row and its result is not stored.
// With router_halves = 2 a unit is one half of a tile's K blocks (units
// u and u + tiles are the two halves of tile u), stored as partial logits in
// the half's own array; the top-k adds the two in half order.
// tile: kRouterTileBytes of LDS.
constexpr int kRouterSplitTiles = 128;  // router_mfma splits K up to this many 16 x 16 tiles
__device__ __forceinline__ int router_halves(const Params& P) {
  // At most 128 tiles (half a grid of one workgroup per CU): without the
  // split half of the grid has no unit and the logits wait for the other half
  // (T=128: ~30 us, one tile's 0.7 MB at one CU's share of the bandwidth).
  // The choice depends on the shape only, so that the logits (and every
  // result after them) are the same on any grid.
  if (P.T <= kRouterMfmaT) return 1;
  return ((P.E + 15) / 16) * ((P.T + 15) / 16) <= kRouterSplitTiles ? 2 : 1;
}
// TB = 2 where there are at least 512 16 x 16 tiles: a unit covers 32 tokens
// (two 16-token blocks sharing each W_r load), so W_r is read T/32 instead of
// T/16 times (T=512: 1.4 instead of 2.1 MB per workgroup, the step being
// bound by these reads).  Shape only, as router_halves.
__device__ __forceinline__ int router_token_blocks(const Params& P) {
  if (P.T <= kRouterMfmaT) return 1;
  return ((P.E + 15) / 16) * ((P.T + 15) / 16) >= 4 * kRouterSplitTiles ? 2 : 1;
}
// One unit: experts e0 .. e0 + 15, tokens t0 .. t0 + 16 TB - 1, K blocks
// [kb0, kb1) of this wave; partial logits of half h.  All threads.
template <int TB>
__device__ __forceinline__ void router_unit(const Params& P, uint32_t tag, int e0, int t0, int h, int kb0, int kb1,
                                            float* tile) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int E2 = (P.E + 1) & ~1;
  const int r = lane & 15, q = lane >> 4;
  const f32x4_t* w = reinterpret_cast<const f32x4_t*>(P.wr + (size_t)min(e0 + r, P.E - 1) * P.d) + q;
  const uint2* xr[TB];
#pragma unroll
  for (int bb = 0; bb < TB; ++bb)
    xr[bb] = reinterpret_cast<const uint2*>(P.x + (size_t)min(t0 + 16 * bb + r, P.T - 1) * P.d) + q;
  // K blocks in groups of kRB, the next group's loads in flight while the
  // current one runs (blocks past kb1 re-read block kb1 - 1 and are skipped)
  // four accumulators per token block (one per MFMA step), so that
  // consecutive MFMAs do not wait for each other's results; added at the end
  constexpr int kRB = 8;
  f32x4_t acc4[TB][4];
#pragma unroll
  for (int bb = 0; bb < TB; ++bb)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) acc4[bb][s4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t a[2][kRB];
  uint2 b[2][TB][kRB];
  const auto load = [&](int g, int j0) {
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      const int j = min(j0 + i, kb1 - 1);
      a[g][i] = w[4 * j];
#pragma unroll
      for (int bb = 0; bb < TB; ++bb) b[g][bb][i] = xr[bb][4 * j];
    }
  };
  const auto run = [&](int g, int j0) {
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      if (j0 + i < kb1) {  // uniform
#pragma unroll
        for (int bb = 0; bb < TB; ++bb) {
          acc4[bb][0] = mfma_f32(a[g][i].x, bf16lo(b[g][bb][i].x), acc4[bb][0]);
          acc4[bb][1] = mfma_f32(a[g][i].y, bf16hi(b[g][bb][i].x), acc4[bb][1]);
          acc4[bb][2] = mfma_f32(a[g][i].z, bf16lo(b[g][bb][i].y), acc4[bb][2]);
          acc4[bb][3] = mfma_f32(a[g][i].w, bf16hi(b[g][bb][i].y), acc4[bb][3]);
        }
      }
    }
  };
  if (kb1 > kb0) {
    load(0, kb0);
    for (int j = kb0; j < kb1; j += 2 * kRB) {
      load(1, j + kRB);
      run(0, j);
      if (j + kRB >= kb1) break;
      load(0, j + 2 * kRB);
      run(1, j + kRB);
    }
  }
#pragma unroll
  for (int bb = 0; bb < TB; ++bb) {
    const f32x4_t acc = (acc4[bb][0] + acc4[bb][1]) + (acc4[bb][2] + acc4[bb][3]);
    // D row = expert 4q + i, column = token r
#pragma unroll
    for (int i = 0; i < 4; ++i) tile[wave * 256 + (4 * q + i) * 16 + r] = acc[i];
    __syncthreads();
    if (threadIdx.x < 256) {
      const int ei = threadIdx.x >> 4, ti = threadIdx.x & 15, t = t0 + 16 * bb + ti;
      float l = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) l += tile[v * 256 + ei * 16 + ti];
      if (e0 + ei < P.E && t < P.T)
        st_tagged(&P.lgp[((size_t)h * P.T + t) * E2 + e0 + ei], __builtin_bit_cast(uint32_t, l), tag);
    }
    __syncthreads();
  }
}
__device__ __forceinline__ void router_mfma(const Params& P, uint32_t tag, int wg, int G, float* tile) {
  const int wave = threadIdx.x / kWave;
  const int tb = router_token_blocks(P), hs = router_halves(P);
  const int ne16 = (P.E + 15) / 16, ntb = ((P.T + 15) / 16 + tb - 1) / tb, tiles = ne16 * ntb;
  const int nkb = P.d / 16;
  for (int u = wg; u < tiles * hs; u += G) {
    const int tu = u % tiles, h = u / tiles;
    const int e0 = (tu / ntb) * 16, t0 = (tu % ntb) * 16 * tb;
    const int hb0 = h * nkb / hs, hn = (h + 1) * nkb / hs - hb0;
    const int kb0 = hb0 + wave * hn / kWaves, kb1 = hb0 + (wave + 1) * hn / kWaves;
    if (tb == 2)  // uniform
      router_unit<2>(P, tag, e0, t0, h, kb0, kb1, tile);
    else
      router_unit<1>(P, tag, e0, t0, h, kb0, kb1, tile);
  }
}

template <bool XLDS, class Pre>
__device__ __forceinline__ void router_step(const Params& P, const Smem& S, uint32_t tag, int wg, int G, Pre pre) {
  __shared__ float s_part[kWaves][kRouterTok];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int ngr = (P.T + kRouterTok - 1) / kRouterTok;
  const int nunits = P.E * ngr;
  const int dw = P.d / kWaves;  // a multiple of 4 (d is a multiple of 32)
  const int n4 = dw / 4;        // <= kRouterF4 * kWave
  const int NCH = P.d / 32;
  const int E2 = (P.E + 1) & ~1;
  bool first = true;
  for (int u = wg; u < nunits; u += G) {
    const int e = u / ngr, g = u % ngr;
    const int t0 = g * kRouterTok, nt = min(kRouterTok, P.T - t0);
    const int c0 = wave * dw;
    const f32x4_t* w = reinterpret_cast<const f32x4_t*>(P.wr + (size_t)e * P.d + c0);
    f32x4_t wv[kRouterF4];
#pragma unroll
    for (int i = 0; i < kRouterF4; ++i) {
      const int c = lane + kWave * i;
      const f32x4_t v = w[min(c, n4 - 1)];  // tail lanes re-read a valid chunk and get a zero weight
      wv[i] = c < n4 ? v : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (first) {
      pre();
      first = false;
    }
    float acc[kRouterTok];
#pragma unroll
    for (int j = 0; j < kRouterTok; ++j) {
      acc[j] = 0.f;
      if (j < nt) {  // uniform
#pragma unroll
        for (int i = 0; i < kRouterF4; ++i) {
          const int col = c0 + 4 * min(lane + kWave * i, n4 - 1);
          uint2 xv;
          if (XLDS) {
            const int ch = col / 32, q = (col % 32) / 8, half = (col % 8) / 4;
            xv = reinterpret_cast<const uint2*>(S.xs)[((size_t)(t0 + j) * 4 * NCH + q * NCH + ch) * 2 + half];
          } else {
            xv = *reinterpret_cast<const uint2*>(P.x + (size_t)(t0 + j) * P.d + col);
          }
          acc[j] = fmaf(wv[i].x, bf16lo(xv.x), acc[j]);
          acc[j] = fmaf(wv[i].y, bf16hi(xv.x), acc[j]);
          acc[j] = fmaf(wv[i].z, bf16lo(xv.y), acc[j]);
          acc[j] = fmaf(wv[i].w, bf16hi(xv.y), acc[j]);
        }
      }
    }
    const float s = reduce8(acc);  // lanes 8j..8j+7: token j's sum over this wave's columns
    if ((lane & 7) == 0) s_part[wave][lane >> 3] = s;
    __syncthreads();
    if (wave == 0 && lane < nt) {
      float l = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) l += s_part[v][lane];
      st_tagged(&P.lgp[(size_t)(t0 + lane) * E2 + e], __builtin_bit_cast(uint32_t, l), tag);
    }
    __syncthreads();
  }
  if (first) pre();
}

// ---------------------------------------------------------------- top-k -----
// One wave, token t: gathers the tagged logits, selects the k largest in
// (logit desc, expert asc) order and their softmax over the selected set
// ([P3-FP4] top-k routing).  Lane j < k returns expert j and gate j.
// Returns false if the wait was abandoned.  Lane L holds the logits of
// experts 2(L + 64m) + b in v[2m + b] (one 16-byte load per pair).
// VPL: logits per lane (E <= 64 * VPL).
template <int VPL>
__device__ __forceinline__ bool topk_token(const Params& P, uint32_t tag, int t, int hs, int* out_i, float* out_w,
                                           bool debug) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t want = tag + P.withhold;
  const int E2 = (P.E + 1) & ~1, np = E2 / 2;
  float v[VPL];
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(P.lgp + (size_t)t * E2, (uint32_t)E2 * 8u);
  // the second half's partial logits (router_halves = 2), else unused
  const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(P.lgp + ((size_t)(hs - 1) * P.T + t) * E2, (uint32_t)E2 * 8u);
  const uint64_t t0 = wall_clock64();
  int round = 0;
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int m = 0; m < VPL / 2; ++m) {
      v[2 * m] = v[2 * m + 1] = 0.f;
      if (kWave * m < np) {  // uniform
        const int p = lane + kWave * m;
        const u32x4_t q = ld_coherent16(rs, (uint32_t)min(p, np - 1) * 16u);
        if (2 * p < P.E) {
          ok &= q.y == want;
          v[2 * m] = u2f(q.x);
        }
        if (2 * p + 1 < P.E) {
          ok &= q.w == want;
          v[2 * m + 1] = u2f(q.z);
        }
        if (hs == 2) {  // uniform: logit = first half + second half
          const u32x4_t q2 = ld_coherent16(rs2, (uint32_t)min(p, np - 1) * 16u);
          if (2 * p < P.E) {
            ok &= q2.y == want;
            v[2 * m] = v[2 * m] + u2f(q2.x);
          }
          if (2 * p + 1 < P.E) {
            ok &= q2.w == want;
            v[2 * m + 1] = v[2 * m + 1] + u2f(q2.z);
          }
        }
      }
    }
    if (__all(ok)) break;
    if (!keep_waiting(P, tag, t0, kSiteLogits, t, round, 0)) return false;  // few waves poll: short sleeps
  }
  if (debug) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = 2 * (lane + kWave * (i / 2)) + (i & 1);
      if (e < P.E) P.logits[(size_t)t * P.E + e] = v[i];
    }
  }
  // (logit desc, expert asc) as one 64-bit key: order-preserving logit bits
  // (-0 taken as +0) above the complemented expert index; 0 = no candidate.
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = 2 * (lane + kWave * (i / 2)) + (i & 1);
    const uint32_t b = __builtin_bit_cast(uint32_t, v[i] + 0.f);
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    key[i] = e < P.E ? ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)e : 0ull;
  }
  // each lane keeps its largest remaining key; a round takes the wave maximum
  // and only the lane that held it (keys are distinct) looks for its next one
  uint64_t lb = 0, mine = 0, top = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (kWave * (i / 2) < np) lb = max_u64(lb, key[i]);  // uniform guard
  for (int j = 0; j < P.k; ++j) {
    const uint64_t best = wave_max_u64(lb);
    if (lb == best) {
      uint64_t nb = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        if (kWave * (i / 2) < np) {
          if (key[i] == best) key[i] = 0ull;
          nb = max_u64(nb, key[i]);
        }
      }
      lb = nb;
    }
    if (j == 0) top = best;
    if (lane == j) mine = best;
  }
  auto key_value = [](uint64_t kk) {
    const uint32_t o = (uint32_t)(kk >> 32);
    return u2f((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
  };
  const float my_v = key_value(mine), vmax = key_value(top);
  const int my_i = (int)~(uint32_t)mine;
  const float ex = (lane < P.k) ? expf(my_v - vmax) : 0.f;
  const float z = wave_sum(ex);
  *out_i = my_i;
  *out_w = ex / z;
  return true;
}

// Token t's top-k is computed by one wave (the owner) and published as
// tagged records in kTopkRep copies; every workgroup then reads the copy
// wg % kTopkRep.  Publishing 16 bytes per slot instead of having every
// workgroup gather all T*E logits keeps the many-reader traffic off the few
// memory channels that hold the logits.  Owners: for T <= NW, waves
// t * NW / T (spread over the grid), else waves t mod NW.
__device__ __forceinline__ bool topk_publish(const Params& P, uint32_t tag, int gw, int NW) {
  const int lane = threadIdx.x & (kWave - 1);
  const int T = P.T, TK = P.T * P.k;
  int t = T <= NW ? (int)(((int64_t)gw * T + NW - 1) / NW) : gw;
  if (T <= NW && (t >= T || (int)((int64_t)t * NW / T) != gw)) return true;
  const int hs = router_halves(P);
  for (; t < T; t += NW) {
    int ii;
    float ww;
    const bool ok = P.E <= 4 * kWave ? topk_token<4>(P, tag, t, hs, &ii, &ww, true)
                                     : topk_token<kMaxE / kWave>(P, tag, t, hs, &ii, &ww, true);
    if (!ok) return false;
    if (lane < P.k) {
      const uint32_t wb = __builtin_bit_cast(uint32_t, ww);
#pragma unroll
      for (int r = 0; r < kTopkRep; ++r) {
        uint64_t* rec = P.tk + ((size_t)r * TK + (size_t)t * P.k + lane) * 2;
        st_tagged(rec, (uint32_t)ii, tag);
        st_tagged(rec + 1, wb, tag);
      }
    }
    if (T <= NW) break;
  }
  return true;
}

// Copy all top-k records of copy `rep` into LDS (waits for them).  All
// threads; each wave polls only its own slots.
__device__ __forceinline__ bool load_topk(const Params& P, const Smem& S, uint32_t tag, int rep) {
  const int TK = P.T * P.k;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(P.tk + (size_t)rep * TK * 2, (uint32_t)TK * 16u);
  bool ok = true;
  const uint64_t t0 = wall_clock64();
  int round = 0;
  for (int base = 0; base < TK && ok; base += kWG) {
    const int s = base + threadIdx.x;
    for (;;) {
      bool ready = true;
      if (s < TK) {
        const u32x4_t q = ld_coherent16(rs, (uint32_t)s * 16u);
        ready = q.y == tag && q.w == tag;
        if (ready) {
          S.tki[s] = (int)q.x;
          S.tkw[s] = u2f(q.z);
        }
      }
      if (__all(ready)) break;
      if (!keep_waiting(P, tag, t0, kSiteTopk, base, round, 1)) {
        ok = false;
        break;
      }
    }
  }
  return ok;
}

// ---------------------------------------------------------- permutation -----
// Pairs (token t, slot j) ordered by (expert asc, token asc): one bit per
// (expert, token) set with an LDS atomic OR (order independent); the rank of
// a pair in its expert's list is the number of set bits below its token.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int s = scratch[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Work model of the expert steps, per row of an expert with n tokens (from
// per-workgroup timings on MI355X): a gate/up row pair costs 16 + 5 per extra
// token (the weights are read once, the dot products repeat) + 4 per extra
// group of g tokens (g = kGUTok of the variant: the row pair is decoded again
// for each group; the term took the shared-routing 8-token block, with up to
// 7 tokens per expert, from 188.4 to 184.7 us and left the others unchanged);
// a W_down row costs 10 per pass over the row plus 4 for the second token of
// a two-token pass (F <= 2048 takes tokens two at a time).
__device__ __forceinline__ int gu_cost(int n, int g) { return 16 + 5 * (n - 1) + 4 * ((n + g - 1) / g - 1); }
__device__ __forceinline__ int dn_cost(int n, int F) { return F <= 2048 ? 14 * (n / 2) + 10 * (n % 2) : 10 * n; }

// Work model of the MFMA path, per workgroup unit of an expert with n tokens,
// in one scale for both steps (a workgroup's down units are dealt by its
// gate/up work, see order_down): a
// pass over a gate/up unit (128 rows each of W_gate and W_up, 128 d bytes of
// codes) costs 7 d / 256 with one column group of 16 tokens and 8 d / 256
// with two; a pass over a down unit (512 rows of W_down, 256 F bytes) costs
// 16 F / 256 with one group and 22 F / 256 with two.  Fitted to per-workgroup
// timings on MI355X at T=128 and T=512 (d=7168, ffn=2048): a gate/up unit
// pass took 50 / 57 us, a down unit pass 31-36 / 43-45 us.
__device__ __forceinline__ int gu_cost_mfma(int n, int d) {
  const int s = (d + 255) / 256;
  int c = 0;
  for (int p = 0; p < n; p += kGUPass) c += s * (6 + (min(kGUPass, n - p) + 15) / 16);
  return c;
}
__device__ __forceinline__ int dn_cost_mfma(int n, int F) {
  const int s = (F + 255) / 256;
  int c = 0;
  for (int p = 0; p < n; p += kDnPass) c += s * (10 + 6 * ((min(kDnPass, n - p) + 15) / 16));
  return c;
}


// MFMA path: the position of workgroup j among the XCD's per workgroups in
// the order of their modelled gate/up work (least first, ties to the lower
// index; workgroup i takes gate/up units S.misc[5] + i, + per, ... below
// S.misc[3]).  The down units are dealt in turn in this order, so the
// workgroups with less gate/up work take the down units left over after the
// last full turn and start the turns first.  Dealt in turn by index instead,
// the workgroups that ended the gate/up step last also took the extra down
// units: at T=128 with Zipf routing the modelled shares explained the
// per-workgroup times (correlation 0.96-0.97) and the layer ended ~100 us
// after the median workgroup.  Wave 0; per <= 64.
__device__ __forceinline__ int order_down(const Smem& S, int per, int j, int Rg) {
  const int lane = threadIdx.x & (kWave - 1);
  int w = 0x7FFFFFFF;  // lanes past per: after every workgroup
  {
    const int g1 = uni(S.misc[3]);
    int u = uni(S.misc[5]) + lane;
    if (lane < per) {
      w = 0;
      if (u < g1) {
        int a = u / Rg, rem = u - a * Rg;
        while (u < g1) {
          w += S.cgu[a + 1] - S.cgu[a];
          u += per;
          rem += per;
          while (rem >= Rg) {
            rem -= Rg;
            ++a;
          }
        }
      }
    }
  }
  const int wj = __builtin_amdgcn_readlane(w, j);
  return __popcll(__ballot(w < wj)) + __popcll(__ballot(w == wj) & ((1ull << j) - 1ull));
}

// Index, in the (active expert, row) list with R rows per expert, of the
// first row whose modelled start lies at or after work position c (c in
// [0, R * cum[na]]).  cum: cumulative work per row of the active experts.
__device__ __forceinline__ int row_at(const int* cum, int na, int R, int w, int G) {
  // Work position c = floor(R * cum[na] * w / G).  A full wave searches
  // together for the last active expert starting at or below c: the lanes
  // sample every 16th entry, then the 17 entries after the last sample at or
  // below c / R (cum is strictly increasing over [0, na], na <= 1024).
  // Quotients of exact integers below 2^53 are taken in double precision: the
  // distance of a non-integer quotient to the next integer is at least 1/G,
  // far above the rounding error, so the floors are exact.
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t X = (int64_t)uni(cum[na]) * w;
  // G is a power of two in the launches the library makes (a grid of one
  // workgroup per CU, times the rounds): then the floors are shifts
  const bool pow2 = (G & (G - 1)) == 0;
  const int sh = __builtin_ctz((unsigned)G);
  const auto fdiv = [&](int64_t v) { return pow2 ? (int)(v >> sh) : (int)floor((double)v / (double)G); };
  const int cq = fdiv(X);  // floor(c / R)
  const uint64_t b1 = __ballot(cum[min(lane * 16, na)] <= cq);  // a prefix of the lanes, lane 0 set
  const int L = 63 - __clzll(b1);
  const int i2 = min(L * 16 + lane, na);
  const uint64_t b2 = __ballot(lane <= 16 && cum[i2] <= cq);
  const int lo = min(L * 16 + 63 - __clzll(b2), na);
  if (lo >= na) return na * R;
  const int c0 = uni(cum[lo]);
  const int u = uni(cum[lo + 1]) - c0;
  // c - R * cum[lo] = floor(R * (X - G * cum[lo]) / G), with 0 <= X - G * cum[lo] < G * u
  const int64_t t = (int64_t)R * (X - (int64_t)G * c0);
  const int rem = fdiv(t);
  const int i = (rem + u - 1) / u;
  return lo * R + min(i, R);
}

// Rows [q0, q1) of part w of W: equal shares of the modelled work.  One wave.
__device__ __forceinline__ void work_range(const int* cum, int na, int R, int w, int W, int& q0, int& q1) {
  q0 = row_at(cum, na, R, w, W);
  q1 = row_at(cum, na, R, w + 1, W);
}

// T*k <= 64: wave 0 alone, one pair per lane.  The position of pair s is the
// number of pairs of a lower expert plus the pairs of the same expert in lower
// slots (each token picks an expert once, so lower slot = lower token).
// Writes what build_perm writes; S.off holds the offsets of the active experts
// and of the entry after each (the only ones read).  All threads.
__device__ __forceinline__ void build_perm_wave(const Params& P, const Smem& S, bool debug) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int E = P.E, TK = P.T * P.k;
  __syncthreads();
  if (tid < kWave) {
    const bool valid = lane < TK;
    const int e = valid ? S.tki[lane] : 0x7FFFFFFF;
    // rank by expert with ballots over the expert index bits (MSB first):
    // `eq` keeps the lanes whose bits so far equal this lane's
    const int nb = 32 - __clz(max(E - 1, 1));
    uint64_t eq = __ballot(valid);
    int lower = 0;
    for (int b = nb - 1; b >= 0; --b) {
      const uint64_t ones = __ballot(valid && ((e >> b) & 1));
      if ((e >> b) & 1) {
        lower += __popcll(eq & ~ones);
        eq &= ones;
      } else {
        eq &= ~ones;
      }
    }
    const int before = __popcll(eq & ((1ull << lane) - 1ull));
    const int same = __popcll(eq);
    const int pos = lower + before;
    const bool first = valid && before == 0;
    // mark the first position of every expert, read the marks back as a mask
    if (valid) {
      S.slot[pos] = lane;
      S.cdn[pos] = first ? 1 : 0;  // scratch until the work model below
    }
    const uint64_t fm = __ballot(valid && S.cdn[lane] != 0);
    const int a = __popcll(fm & ((1ull << (pos - before)) - 1ull));  // distinct experts below e
    const int na = __popcll(fm);
    if (first) {
      S.act[a] = e;
      S.off[e] = pos;
      S.off[e + 1] = pos + same;  // equal to the next active expert's offset if it is e + 1
      S.cgu[a] = same;            // token counts by active index, read back below
    }
    if (lane == 0) S.misc[0] = na;
    const int n = lane < na ? S.cgu[lane] : 0;
    const int g = lane < na ? (P.mfma ? gu_cost_mfma(n, P.d) : gu_cost(n, P.xmode ? kGUTok<true> : kGUTok<false>)) : 0;
    const int dc = lane < na ? (P.mfma ? dn_cost_mfma(n, P.F) : dn_cost(n, P.F)) : 0;
    const int gi = wave_inclusive_scan(g), di = wave_inclusive_scan(dc);
    if (lane < na) {
      S.cgu[lane] = gi - g;
      S.cdn[lane] = di - dc;
    }
    if (lane == na - 1) {
      S.cgu[na] = gi;
      S.cdn[na] = di;
    }
    if (debug) {
      if (valid) {
        P.pos[lane] = pos;
        P.sorted_slot[pos] = lane;
        P.topk_idx[lane] = e;
        P.topk_w[lane] = S.tkw[lane];
      }
      if (first) P.active[a] = e;
      if (lane == 0) *P.n_active = na;
      for (int eb = 0; eb <= E; eb += kWave) {
        const int ee = eb + lane;
        int c = 0;
        for (int j = 0; j < TK; ++j) c += S.tki[j] < ee;
        if (ee <= E) P.offsets[ee] = c;
      }
    }
  }
  __syncthreads();
}

// All threads of the workgroup.  Reads S.tki / S.tkw, writes S.off / S.slot /
// S.act / S.misc[0] and the work model; `debug` also writes the plain copies
// to global memory.
__device__ __forceinline__ void build_perm(const Params& P, const Smem& S, bool debug) {
  if (P.T * P.k <= kWave) {
    build_perm_wave(P, S, debug);
    return;
  }
  const int tid = threadIdx.x;
  const int W = (P.T + 63) / 64;
  const int E = P.E, TK = P.T * P.k;
  uint64_t* mask = S.mask;
  __syncthreads();
  for (int i = tid; i < E * W; i += kWG) mask[i] = 0ull;
  __syncthreads();
  for (int s = tid; s < TK; s += kWG) {
    const int t = s / P.k, e = S.tki[s];
    atomicOr(reinterpret_cast<unsigned long long*>(&mask[(size_t)e * W + t / 64]), 1ull << (t & 63));
  }
  __syncthreads();
  // counts and exclusive scans over experts, two experts per thread (E <= 1024)
  const int e0 = tid * 2;
  int c2[2], a2[2], csum = 0, asum = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = e0 + i;
    int c = 0;
    if (e < E)
      for (int w = 0; w < W; ++w) c += __popcll(mask[(size_t)e * W + w]);
    c2[i] = c;
    a2[i] = c > 0;
    csum += c;
    asum += a2[i];
  }
  int ctot, atot;
  int cbase = block_exclusive_scan(csum, S.misc + 8, &ctot);
  int abase = block_exclusive_scan(asum, S.misc + 8, &atot);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = e0 + i;
    if (e < E) {
      S.off[e] = cbase;
      if (a2[i]) S.act[abase] = e;
      if (debug) {
        P.offsets[e] = cbase;
        if (a2[i]) P.active[abase] = e;
      }
    }
    cbase += c2[i];
    abase += a2[i];
  }
  if (tid == 0) {
    S.off[E] = ctot;
    S.misc[0] = atot;
    if (debug) {
      P.offsets[E] = ctot;
      *P.n_active = atot;
    }
  }
  __syncthreads();
  {
    // cumulative modelled work of the active experts (see gu_cost, dn_cost)
    const int na = S.misc[0];
    int g2[2], d2[2], gs = 0, ds = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int a = e0 + i;
      const int n = a < na ? S.off[S.act[a] + 1] - S.off[S.act[a]] : 0;
      g2[i] = a < na ? (P.mfma ? gu_cost_mfma(n, P.d) : gu_cost(n, P.xmode ? kGUTok<true> : kGUTok<false>)) : 0;
      d2[i] = a < na ? (P.mfma ? dn_cost_mfma(n, P.F) : dn_cost(n, P.F)) : 0;
      gs += g2[i];
      ds += d2[i];
    }
    int gt, dt;
    int gb = block_exclusive_scan(gs, S.misc + 8, &gt);
    int db = block_exclusive_scan(ds, S.misc + 8, &dt);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int a = e0 + i;
      if (a < na) {
        S.cgu[a] = gb;
        S.cdn[a] = db;
      }
      gb += g2[i];
      db += d2[i];
    }
    if (tid == 0) {
      S.cgu[na] = gt;
      S.cdn[na] = dt;
    }
  }
  for (int s = tid; s < TK; s += kWG) {
    const int t = s / P.k, e = S.tki[s];
    const uint64_t* me = mask + (size_t)e * W;
    int r = 0;
    for (int w = 0; w < t / 64; ++w) r += __popcll(me[w]);
    r += __popcll(me[t / 64] & ((1ull << (t & 63)) - 1ull));
    const int p = S.off[e] + r;
    S.slot[p] = s;
    if (debug) {
      P.pos[s] = p;
      P.sorted_slot[p] = s;
      P.topk_idx[s] = e;
      P.topk_w[s] = S.tkw[s];
    }
  }
  __syncthreads();
}

// ----------------------------------------------------- x into LDS -----------
// Token rows of x in a piece-transposed layout: 16-byte piece q (elements
// 8q..8q+7) of chunk c (elements 32c..32c+31) of row r at index
// r*4*NCH + q*NCH + c, so lanes reading consecutive chunks hit consecutive
// LDS addresses.  `tok(r)` maps a staged row to a token.
template <class TokOf>
__device__ __forceinline__ void stage_x(const Params& P, u32x4_t* xs, int nrows, TokOf tok) {
  const int NCH = P.d / 32, per = 4 * NCH;
  const int n = nrows * per;
  constexpr int U = 4;
  for (int base = 0; base < n; base += kWG * U) {
    u32x4_t v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int i = min(base + j * kWG + (int)threadIdx.x, n - 1);
      const int r = i / per, rem = i % per, c = rem / 4, q = rem % 4;
      v[j] = *reinterpret_cast<const u32x4_t*>(P.x + (size_t)tok(r) * P.d + (size_t)c * 32 + q * 8);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int i = base + j * kWG + (int)threadIdx.x;
      if (i < n) {
        const int r = i / per, rem = i % per, c = rem / 4, q = rem % 4;
        xs[r * per + q * NCH + c] = v[j];
      }
    }
  }
}

// ------------------------------------------------- gate/up + SwiGLU ---------
// Row pair i of expert e ([P5-FP4] gate_proj, up_proj): g = W_gate[i] . x_t,
// u = W_up[i] . x_t for every token t routed to e, h = silu(g) * u.

struct GURow {
  u32x4_t g[kGUChunks], u[kGUChunks];
  uint32_t sg[kGUChunks], su[kGUChunks];
};

// Loads are unconditional (no divergent branch between them, so they all stay
// in flight): a lane past the end of the row re-reads the row's last chunk
// with its scale byte masked to 0, which decodes as 2^-127 (see e8m0_to_f32).
// Its 32 terms then add less than 2^-110 for |x| < 2^8, below half an ulp of
// any fp32 sum above 2^-86 in magnitude: they do not change g or u.  (Zeroing the codes instead cost 2% of the
// verify layer's time.)
__device__ __forceinline__ void gu_load(const Params& P, const Smem& S, int rho, GURow& R) {
  const int lane = threadIdx.x & (kWave - 1);
  const int d = P.d, F = P.F, NCH = d / 32;
  const int a = uni(rho / F), i = uni(rho % F);
  const int e = uni(S.act[a]);
  const size_t pbytes = (size_t)3 * d * F / 2, sbytes = (size_t)3 * d * F / 32;
  const uint8_t* pg = P.packed + (size_t)e * pbytes + (size_t)i * (d / 2);
  const uint8_t* pu = pg + (size_t)F * d / 2;
  const uint8_t* sg = P.scales + (size_t)e * sbytes + (size_t)i * NCH;
  const uint8_t* su = sg + (size_t)F * NCH;
#pragma unroll
  for (int m = 0; m < kGUChunks; ++m) {
    const int c = lane + kWave * m;
    const int cc = min(c, NCH - 1);
    R.g[m] = ld_stream16(pg + cc * 16);
    R.u[m] = ld_stream16(pu + cc * 16);
    const uint32_t keep = c < NCH ? 0xFFu : 0u;
    R.sg[m] = sg[cc] & keep;
    R.su[m] = su[cc] & keep;
  }
}

__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.f + expf(-g)) * u; }

// Order of a pair's F tagged h words on the small-batch path with x of every
// token in LDS (xmode 0, chunk-major): value i (chunk c = i / 32, element
// e = i % 32 of it) is word 2 ((e / 2) NCH + c) + e % 2, so 16-byte piece
// v NCH + c holds values 32 c + 2 v and 32 c + 2 v + 1.  A wave whose lane c
// needs chunk c (the down step) then reads NCH consecutive pieces per load
// instruction (1 KiB at F = 2048) instead of one piece 256 bytes apart per
// lane.  Measured on MI355X, 8 tokens: -1% per layer (gate/up +2 us for its
// scattered 8-byte stores, down -4 us).  With more tokens (xmode 1, more h
// stores per row) the stores cost more than the loads save (16 tokens: +3%),
// so there, and on the MFMA path, h stays in value order ([pair][F]).
__device__ __forceinline__ int h_word(int i, int nch) { return 2 * (((i & 31) >> 1) * nch + (i >> 5)) + (i & 1); }

// Small batches: x in LDS (xmode 0: row t = token t; xmode 1: row r = pair
// xbase + r, see stage_pairs).  Each chunk of the row pair is decoded once and
// used for up to kGUTok tokens.  A token group whose pairs are not in LDS
// (xmode 1, more pairs in the workgroup's range than LDS rows) reads x from
// global memory instead: correct, slower.
template <bool XP>
__device__ __forceinline__ void gu_compute_resident(const Params& P, const Smem& S, uint32_t tag, int rho,
                                                    const GURow& R) {
  const int lane = threadIdx.x & (kWave - 1);
  const int NCH = P.d / 32;
  const int a = uni(rho / P.F), i = uni(rho % P.F);
  const int e = uni(S.act[a]);
  const int p0 = uni(S.off[e]), ne = uni(S.off[e + 1]) - p0;
  const int xb0 = XP ? uni(S.misc[kMiscXBase]) : 0, xn = XP ? uni(S.misc[kMiscXRows]) : 0;
  const auto group = [&](int tb, auto global_x) {
    constexpr bool GX = decltype(global_x)::value;
    const int nb = min(kGUTok<XP>, ne - tb);
    float g[kGUTok<XP>], u[kGUTok<XP>];
    int xrow[kGUTok<XP>];
#pragma unroll
    for (int t = 0; t < kGUTok<XP>; ++t) {
      g[t] = u[t] = 0.f;
      const int pr = p0 + tb + t;
      xrow[t] = t < nb ? (GX || !XP ? uni(S.slot[pr]) / P.k : pr - xb0) : 0;
    }
#pragma unroll
    for (int m = 0; m < kGUChunks; ++m) {
      if (kWave * m < NCH) {  // uniform; lanes past the row end have scale byte 0 (gu_load)
        bf16x2_t dg[16], du[16];
        decode32_bf16(R.g[m], e8m0_to_f32(R.sg[m]), dg);
        decode32_bf16(R.u[m], e8m0_to_f32(R.su[m]), du);
        const int cc = min(lane + kWave * m, NCH - 1);
#pragma unroll
        for (int t = 0; t < kGUTok<XP>; ++t) {
          if (t < nb) {
            u32x4_t xq[4];
            if (GX) {
              const u32x4_t* xg = reinterpret_cast<const u32x4_t*>(P.x + (size_t)xrow[t] * P.d) + 4 * cc;
#pragma unroll
              for (int q = 0; q < 4; ++q) xq[q] = xg[q];
            } else {
              const u32x4_t* xb = S.xs + (size_t)xrow[t] * 4 * NCH;
#pragma unroll
              for (int q = 0; q < 4; ++q) xq[q] = xb[q * NCH + cc];
            }
            g[t] = dot32_bf16_dec(dg, xq, g[t]);
            u[t] = dot32_bf16_dec(du, xq, u[t]);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kGUTok<XP>; ++t) {
      if (t < nb) {
        const float gs = wave_sum(g[t]), us = wave_sum(u[t]);
        if (lane == 0)
          st_tagged(&P.hq[(size_t)(p0 + tb + t) * P.F + (XP ? i : h_word(i, P.F / 32))],
                    __builtin_bit_cast(uint32_t, swiglu(gs, us)), tag);
      }
    }
  };
  const auto run = [&](int tb) {
    const int nb = min(kGUTok<XP>, ne - tb);
    if (!XP || (p0 + tb >= xb0 && p0 + tb + nb <= xb0 + xn))  // uniform
      group(tb, std::false_type{});
    else
      group(tb, std::true_type{});
  };
  // The first group (usually the only one) outside any loop: a loop whose
  // body reads the row pair's registers makes the compiler wait for every
  // load in flight (vmcnt(0)) at its entry, including the next row pair's.
  run(0);
  for (int tb = kGUTok<XP>; tb < ne; tb += kGUTok<XP>) run(tb);
}

// xmode 1: x rows of the pairs of the experts the workgroup's gate/up range
// touches, as many as the LDS holds (row r = pair xbase + r), into
// S.misc[kMiscXBase] / [kMiscXRows].  After set_ranges (one chunk); all
// threads; ends with a barrier.
__device__ __forceinline__ void stage_pairs(const Params& P, const Smem& S) {
  const int* tab = round_tab(S, 0);
  const int q0 = tab[0], q1 = q0 + tab[kRounds + 1];
  int pb = 0, n = 0;
  if (q1 > q0) {
    const int a0 = q0 / P.F, a1 = (q1 - 1) / P.F;
    pb = S.off[S.act[a0]];
    n = min(S.off[S.act[a1] + 1] - pb, P.xrows);
  }
  if (threadIdx.x == 0) {
    S.misc[kMiscXBase] = pb;
    S.misc[kMiscXRows] = n;
  }
  if (n > 0) stage_x(P, S.xs, n, [&](int r) { return S.slot[pb + r] / P.k; });
  __syncthreads();
}

// Next unit from a workgroup's LDS work counter (one LDS atomic by lane 0).
__device__ __forceinline__ int grab(int* ctr) {
  int v = 0;
  if ((threadIdx.x & (kWave - 1)) == 0) v = atomicAdd(ctr, 1);
  return __builtin_amdgcn_readfirstlane(v);
}

// A wave's walk through its workgroup's chunks (set_ranges): work index j of
// the workgroup (from its LDS counter) is row unit start[k] + j - cum[k] of the
// chunk k with cum[k] <= j < cum[k + 1].  A wave's indices only grow, so the
// chunk only moves forward.
struct Cursor {
  int k, lo, hi, s;
};
__device__ __forceinline__ Cursor cursor_start(const int* tab) {
  return Cursor{0, 0, uni(tab[kRounds + 1]), uni(tab[0])};
}
__device__ __forceinline__ int unit_of(const int* tab, Cursor& c, int j) {
  while (j >= c.hi && c.k < kRounds - 1) {
    ++c.k;
    c.lo = c.hi;
    c.hi = uni(tab[kRounds + c.k + 1]);
    c.s = uni(tab[c.k]);
  }
  return c.s + (j - c.lo);
}

// Each workgroup owns kRounds chunks of the n_active*F row pairs (equal
// shares of the modelled work); its waves take the row pairs one at a time
// from an LDS counter (S.misc[1]), so the two waves that share a SIMD, which
// issue at different rates, finish together.  A wave loads its next row pair
// while computing the current one.
// XP: x rows of the workgroup's pairs in LDS (stage_pairs); else all tokens'.
template <bool XP>
__device__ __forceinline__ void gate_up_waves(const Params& P, const Smem& S, uint32_t tag, int wg, int G) {
  const int* tab = round_tab(S, 0);
  const int Q1 = uni(tab[2 * kRounds]);
  int* ctr = S.misc + 1;
  Cursor cur = cursor_start(tab);
  // Each index is taken one step before its loads are issued, so the LDS
  // atomic's round trip overlaps a compute step; indices only grow, so once
  // one is past the end all later ones are too.
  int j0 = grab(ctr);
  if (j0 >= Q1) return;
  int r0 = unit_of(tab, cur, j0);
  GURow A, B;
  gu_load(P, S, r0, A);
  int j1 = grab(ctr);
  for (;;) {
    // past the end a wave re-reads the row pair it just loaded (cache-hot)
    // and does not use it
    const int r1 = j1 < Q1 ? unit_of(tab, cur, j1) : r0;
    gu_load(P, S, r1, B);
    const int j2 = grab(ctr);
    gu_compute_resident<XP>(P, S, tag, r0, A);
    if (j1 >= Q1) break;
    const int r2 = j2 < Q1 ? unit_of(tab, cur, j2) : r1;
    gu_load(P, S, r2, A);
    const int j3 = grab(ctr);
    gu_compute_resident<XP>(P, S, tag, r1, B);
    if (j2 >= Q1) break;
    r0 = r2;
    j1 = j3;
  }
}

// ------------------------------------------------------------ down ----------
// y_r = W_down[r] . h for every token of expert e ([P5-FP4] down_proj); the
// gated value gate * y_r goes to the token's slot row.  A lane owns MM
// 16-byte chunks of a W_down row and the matching 32*MM values of h per token
// (registers); each step covers kDnRows rows and up to NT tokens.
template <int MM, int ROWS>
struct DnRows {
  u32x4_t w[ROWS][MM];
  uint32_t s[ROWS][MM];
};

template <int MM, int ROWS>
__device__ __forceinline__ void dn_load(const Params& P, int e, int r0, int nr, DnRows<MM, ROWS>& R) {
  const int lane = threadIdx.x & (kWave - 1);
  const int d = P.d, F = P.F, NCH = F / 32;
  const size_t pbytes = (size_t)3 * d * F / 2, sbytes = (size_t)3 * d * F / 32;
  const uint8_t* pd = P.packed + (size_t)e * pbytes + (size_t)F * d + (size_t)r0 * (F / 2);
  const uint8_t* sd = P.scales + (size_t)e * sbytes + (size_t)F * d / 16 + (size_t)r0 * NCH;
#pragma unroll
  for (int j = 0; j < ROWS; ++j) {
    const int jj = min(j, nr - 1);  // rows past the end re-read the last row (not stored)
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const int c = lane + kWave * m;
      const int cc = min(c, NCH - 1);
      R.w[j][m] = ld_stream16(pd + (size_t)jj * (F / 2) + cc * 16);
      R.s[j][m] = sd[(size_t)jj * NCH + cc] & (c < NCH ? 0xFFu : 0u);
    }
  }
}

// h of pair p into registers (the lane's chunks); waits for its tags.  CM:
// chunk-major rows (h_word), else value order.
template <int MM, bool CM>
__device__ __forceinline__ bool dn_load_h(const Params& P, uint32_t tag, int p, float (&h)[MM][32]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int NCH = P.F / 32;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(P.hq + (size_t)p * P.F, (uint32_t)P.F * 8u);
  const uint32_t want = tag + P.withhold_h;
  const uint64_t t0 = wall_clock64();
  // chunk c: 16 pieces NCH pieces apart (CM), else 256 contiguous bytes
  const uint32_t cstride = CM ? 16u : 256u, vstride = CM ? (uint32_t)NCH * 16u : 16u;
  int round = 0;
  // The first attempt reads the whole h at once and through the L2 (it is
  // usually complete by then, and under full load every round trip costs
  // microseconds, an agent-coherent one several times more); later attempts
  // are coherent and first check two words per lane spread over the F rows
  // (512 B per wave per round instead of the whole 8*F bytes).
  const auto read_all = [&]() {
    bool ok = true;
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const int c = lane + kWave * m;
      const uint32_t base = (uint32_t)min(c, NCH - 1) * cstride;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t off = base + (uint32_t)v * vstride;  // values 32 c + 2 v, +1
        const u32x4_t w = round == 0 ? ld_cached16(rs, off) : ld_coherent16(rs, off);
        ok &= (w.y == want) && (w.w == want);
        h[m][2 * v] = c < NCH ? u2f(w.x) : 0.f;
        h[m][2 * v + 1] = c < NCH ? u2f(w.z) : 0.f;
      }
    }
    return __all(ok);
  };
  const uint32_t probe = (uint32_t)min((lane * P.F / kWave) & ~1, P.F - 2) * 8u;
  for (;;) {
    bool go = true;
    if (round > 0) {  // uniform
      const u32x4_t q = ld_coherent16(rs, probe);
      go = __all((q.y == want) && (q.w == want));
    }
    if (go && read_all()) return true;
    if (!keep_waiting(P, tag, t0, kSiteH, p, round, 3)) return false;
  }
}

template <int MM, int NT, int ROWS>
__device__ __forceinline__ void dn_compute(const Params& P, const Smem& S, uint32_t tag, int p0, int ntok, int r0,
                                           int nr, const DnRows<MM, ROWS>& R, const float (&h)[NT][MM][32]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int NCH = P.F / 32;
  float acc[NT][kDnRows];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int j = 0; j < kDnRows; ++j) acc[tt][j] = 0.f;
#pragma unroll
  for (int j = 0; j < ROWS; ++j) {
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      if (kWave * m < NCH) {  // uniform; lanes past the row end have h 0, so they add exactly 0
        float v[32];
        decode32_f32(R.w[j][m], e8m0_to_f32(R.s[j][m]), v);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          if (tt < ntok) acc[tt][j] = dot32(v, &h[tt][m][0], acc[tt][j]);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    if (tt < ntok) {
      const float s = reduce8(acc[tt]);  // lanes 8j..8j+7 hold row j
      const int j = lane >> 3;
      if ((lane & 7) == 0 && j < nr) {
        const int slot = uni(S.slot[p0 + tt]);
        st_tagged(&P.yq[(size_t)slot * P.d + r0 + j], __builtin_bit_cast(uint32_t, S.tkw[slot] * s), tag);
      }
    }
  }
}

// Rows [r, rend) of expert e's W_down against the h of NT-or-fewer pairs
// starting at pair p (ntok of them), ROWS rows per step with the next step's
// rows in flight.
template <int MM, int NT, int ROWS, bool CM>
__device__ __forceinline__ bool down_rows(const Params& P, const Smem& S, uint32_t tag, int e, int p, int ntok, int r,
                                          int rend) {
  float h[NT][MM][32];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    if (tt < ntok) {
      if (!dn_load_h<MM, CM>(P, tag, p + tt, h[tt])) return false;
    }
  }
  DnRows<MM, ROWS> A, B;
  dn_load<MM, ROWS>(P, e, r, min(ROWS, rend - r), A);
  for (; r < rend; r += 2 * ROWS) {
    // prefetches past the segment end re-read its last row and are not used
    const int rB = min(r + ROWS, rend - 1), rA2 = min(r + 2 * ROWS, rend - 1);
    dn_load<MM, ROWS>(P, e, rB, min(ROWS, rend - rB), B);
    dn_compute<MM, NT, ROWS>(P, S, tag, p, ntok, r, min(ROWS, rend - r), A, h);
    dn_load<MM, ROWS>(P, e, rA2, min(ROWS, rend - rA2), A);
    if (r + ROWS < rend) dn_compute<MM, NT, ROWS>(P, S, tag, p, ntok, r + ROWS, min(ROWS, rend - r - ROWS), B, h);
  }
  return true;
}

// F > 2048: each wave streams a contiguous range of the n_active*d rows of
// W_down (equal shares of the modelled work), one token per pass.
template <int MM, bool CM>
__device__ __forceinline__ bool down_waves_static(const Params& P, const Smem& S, uint32_t tag, int gw, int NW) {
  const int d = P.d;
  int q0, q1;
  work_range(S.cdn, uni(S.misc[0]), d, gw, NW, q0, q1);
  int rho = q0;
  while (rho < q1) {
    const int a = uni(rho / d);
    const int seg_end = min(q1, (a + 1) * d);
    const int e = uni(S.act[a]);
    const int p0 = uni(S.off[e]), ne = uni(S.off[e + 1]) - p0;
    const int r0 = rho - a * d, rend = seg_end - a * d;
    for (int tg = 0; tg < ne; ++tg)
      if (!down_rows<MM, 1, 2, CM>(P, S, tag, e, p0 + tg, 1, r0, rend)) return false;
    rho = seg_end;
  }
  return true;
}

// Unit u of the down step: kDnRows consecutive rows of one active expert
// (d / kDnRows units per expert).
__device__ __forceinline__ void dn_unit_rows(const Params& P, const Smem& S, int u, DnRows<1, kDnRows>& R) {
  const int upe = P.d / kDnRows;
  const int a = uni(u / upe);
  dn_load<1, kDnRows>(P, uni(S.act[a]), (u - a * upe) * kDnRows, kDnRows, R);
}

// One unit against every token of its expert, two tokens per pass; the h of
// the pass is kept in registers across units of the same expert.
// HL: h rows staged in LDS by stage_h (row r = pair hb0 + r), read for every
// pass (kept in registers across units it costs more registers than the
// wave has); else each wave loads the h it needs from global memory and keeps
// it across the units of the same expert and token pair.
template <bool HL, bool CM>
__device__ __forceinline__ bool dn_unit_work(const Params& P, const Smem& S, uint32_t tag, int u,
                                             const DnRows<1, kDnRows>& R, float (&h)[2][1][32], int& ha, int& hb,
                                             int hb0) {
  const int lane = threadIdx.x & (kWave - 1);
  const int upe = P.d / kDnRows;
  const int a = uni(u / upe), e = uni(S.act[a]);
  const int p0 = uni(S.off[e]), ne = uni(S.off[e + 1]) - p0;
  const int r = (u - a * upe) * kDnRows;
  for (int tg = 0; tg < ne; tg += 2) {
    const int nt = min(2, ne - tg);
    if (HL) {
      // lanes past the row's chunks (F < 2048) read the last chunk's h; their
      // codes have scale byte 0 (dn_load), 2^-127, which puts their terms far
      // below the rounding of the sums (see gu_load)
      float hl[2][1][32];
      const int nch = P.F / 32, c = min(lane, nch - 1);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int pr = p0 + tg + min(tt, nt - 1);
        if (CM) {
          // chunk-major rows (h_word): lane c reads values 32 c + 2 v, +1 at
          // 8-byte word v NCH + c (consecutive lanes, consecutive words)
          const f32x2_t* hp = reinterpret_cast<const f32x2_t*>(S.xs) + ((size_t)(pr - hb0) * P.F) / 2 + c;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const f32x2_t q = hp[v * nch];
            hl[tt][0][2 * v] = q.x;
            hl[tt][0][2 * v + 1] = q.y;
          }
        } else {
          const f32x4_t* hp =
              reinterpret_cast<const f32x4_t*>(S.xs) + ((size_t)(pr - hb0) * P.F + (size_t)c * 32) / 4;
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            const f32x4_t q = hp[v];
            hl[tt][0][4 * v] = q.x;
            hl[tt][0][4 * v + 1] = q.y;
            hl[tt][0][4 * v + 2] = q.z;
            hl[tt][0][4 * v + 3] = q.w;
          }
        }
      }
      dn_compute<1, 2, kDnRows>(P, S, tag, p0 + tg, nt, r, kDnRows, R, hl);
      continue;
    }
    if (ha != a || hb != tg) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        if (tt < nt && !dn_load_h<1, CM>(P, tag, p0 + tg + tt, h[tt])) return false;
      if (ha < 0) stamp(P, blockIdx.x, 8);  // trace: the first h this wave needs is present
      ha = a;
      hb = tg;
    }
    dn_compute<1, 2, kDnRows>(P, S, tag, p0 + tg, nt, r, kDnRows, R, h);
  }
  return true;
}

// The h of the pairs of the experts the workgroup's down range touches, read
// once by the whole workgroup into LDS (S.xs as floats, row r = pair hb0 + r)
// when they fit in cap_bytes and it pays; the waves then take each pass's h
// from LDS instead of each loading it (coherent 16-byte loads of a ready h
// cost several microseconds under full load, and an expert with more than two
// tokens needs a new h for every pass).  Every wave takes the same decision
// from the LDS tables: `staged` and hb0 out.  When staging, all threads: the
// first barrier orders every wave's last read of x in S.xs before the writes
// of h; ends with a barrier.  False: the wait timed out.
__device__ __forceinline__ bool stage_h(const Params& P, const Smem& S, uint32_t tag, size_t cap_bytes, bool& staged,
                                        int& hb0) {
  __shared__ int s_bad[2], s_go;
  const int* tab = round_tab(S, 1);
  const int q0 = uni(tab[0]), q1 = q0 + uni(tab[kRounds + 1]);
  const int upe = P.d / kDnRows;
  int pb = 0, np = 0, many = 0;
  if (q1 > q0) {
    const int a0 = q0 / upe, a1 = (q1 - 1) / upe;
    pb = uni(S.off[S.act[a0]]);
    np = uni(S.off[S.act[a1] + 1]) - pb;
    for (int a = a0; a <= a1 && !many; ++a) many = S.off[S.act[a] + 1] - S.off[S.act[a]] > 2;
  }
  // Staging costs a workgroup barrier and puts the h latency before the
  // first weight loads; it pays where waves would reload h per pass (an expert
  // with more than two tokens) or have few units to spread their own h loads
  // over (fewer than 16 per wave: measured on MI355X, a threshold of 16
  // took the 4-token verify block from 140 to 137 us and left the 8-token one, at
  // ~26 units per wave, unchanged).
  const bool worth = __builtin_amdgcn_readfirstlane(many) || q1 - q0 < 16 * kWaves;
  staged = worth && np > 0 && (size_t)np * P.F * 4 <= cap_bytes;
  hb0 = pb;
  if (!staged) return true;
  if (threadIdx.x == 0) s_bad[0] = 0;
  __syncthreads();
  float* hl = reinterpret_cast<float*>(S.xs);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(P.hq + (size_t)pb * P.F, (uint32_t)np * (uint32_t)P.F * 8u);
  const int n16 = np * P.F / 2;  // 16-byte pieces of two tagged words
  const uint64_t t0 = wall_clock64();
  for (int round = 0;;) {
    const int par = round & 1;
    if (threadIdx.x == 0) s_bad[par ^ 1] = 0;  // the next round's flag
    bool ok = true;
    for (int i = threadIdx.x; i < n16; i += kWG) {
      // first read through the L2 (dropped of earlier calls' lines, see k_layer)
      const u32x4_t w = round == 0 ? ld_cached16(rs, (uint32_t)i * 16u) : ld_coherent16(rs, (uint32_t)i * 16u);
      if (w.y == tag + P.withhold_h && w.w == tag + P.withhold_h) {
        // the rows keep the order of the tagged words (h_word for xmode 0)
        hl[2 * i] = u2f(w.x);
        hl[2 * i + 1] = u2f(w.z);
      } else {
        ok = false;
      }
    }
    if (!ok) s_bad[par] = 1;
    __syncthreads();
    if (s_bad[par] == 0) return true;  // uniform
    if (threadIdx.x < kWave) {
      int rd = round;
      const bool go = keep_waiting(P, tag, t0, kSiteH, pb, rd, 3);
      if (threadIdx.x == 0) s_go = go ? 1 : 0;
    }
    ++round;
    __syncthreads();
    if (!s_go) return false;
  }
}

// F <= 2048: each workgroup owns a range of the down units (equal shares of
// the modelled work); its waves take units from an LDS counter (S.misc[2])
// and load the next unit's rows while computing the current one.  An
// expert's tokens are taken two at a time, so W_down is read once per two
// tokens.  HL: h from LDS (stage_h).
template <bool HL, bool CM>
__device__ __forceinline__ bool down_loop(const Params& P, const Smem& S, uint32_t tag, int hb0) {
  const int* tab = round_tab(S, 1);
  const int U1 = uni(tab[2 * kRounds]);
  int* ctr = S.misc + 2;
  Cursor cur = cursor_start(tab);
  float h[2][1][32];
  int ha = -1, hb = -1;
  int j0 = grab(ctr);
  if (j0 >= U1) return true;
  int u0 = unit_of(tab, cur, j0);
  DnRows<1, kDnRows> A, B;
  dn_unit_rows(P, S, u0, A);
  int j1 = grab(ctr);  // indices are taken one step ahead (see gate_up_waves)
  for (;;) {
    const int u1 = j1 < U1 ? unit_of(tab, cur, j1) : u0;  // past the end: re-read (cache-hot), unused
    dn_unit_rows(P, S, u1, B);
    const int j2 = grab(ctr);
    if (!dn_unit_work<HL, CM>(P, S, tag, u0, A, h, ha, hb, hb0)) return false;
    if (j1 >= U1) break;
    const int u2 = j2 < U1 ? unit_of(tab, cur, j2) : u1;
    dn_unit_rows(P, S, u2, A);
    const int j3 = grab(ctr);
    if (!dn_unit_work<HL, CM>(P, S, tag, u1, B, h, ha, hb, hb0)) return false;
    if (j2 >= U1) break;
    u0 = u2;
    j1 = j3;
  }
  return true;
}

// HS: the workgroup may stage h in LDS (stage_h; all threads, x_bytes = the x
// area it may use); else every wave loads its own h.  CM: h rows in the
// chunk-major order of h_word (x of every token in LDS), else value order.
template <bool HS, bool CM>
__device__ __forceinline__ bool down_waves_dyn(const Params& P, const Smem& S, uint32_t tag, size_t x_bytes) {
  if (!HS) return down_loop<false, CM>(P, S, tag, 0);
  bool staged;
  int hb0;
  if (!stage_h(P, S, tag, x_bytes, staged, hb0)) return false;
  if (staged) return down_loop<true, CM>(P, S, tag, hb0);  // uniform
  return down_loop<false, CM>(P, S, tag, hb0);
}

template <int MM, bool HS, bool CM>
__device__ __forceinline__ bool down_dispatch(const Params& P, const Smem& S, uint32_t tag, int wg, int G,
                                              size_t x_bytes) {
  if (MM == 1) return down_waves_dyn<HS, CM>(P, S, tag, x_bytes);
  return down_waves_static<MM, CM>(P, S, tag, wg * kWaves + uni(threadIdx.x / kWave), G * kWaves);
}

// The workgroup's share of the expert steps.  Work units: small-batch path,
// gate/up row pairs and kDnRows-row down units; MFMA path, 128-row-pair and
// 512-row units.  Both lists are expert-major over the active experts.
//  - Small-batch path: the gate/up list is cut into kRounds * G chunks of
//    equal modelled work, and workgroup wg owns chunks k * G + wg, k <
//    kRounds, so all workgroups move through the experts together and the h
//    of all but the last round's experts is complete well before the gate/up
//    step ends; the down list is cut into G contiguous ranges (one chunk per
//    workgroup, so a wave rarely needs a new h).  Work tables in round_tab;
//    S.misc[1] / [2] = 0: gate/up and down counters over the workgroup's
//    chunks.
//  - MFMA path: each list is cut into one chunk of equal modelled work per
//    XCD (per workgroups), whose units are dealt in turn: gate/up units U0 +
//    j, U0 + j + per, ... below U1 to workgroup j of the XCD, down units to
//    the workgroups in the order of their modelled gate/up work (order_down).
//    S.misc[5] / [3] = the workgroup's first gate/up unit and U1,
//    S.misc[6] / [4] the same for down, S.misc[kMiscStride] = per.
// All threads; ends with a barrier.
__device__ __forceinline__ void set_ranges(const Params& P, const Smem& S, int wg, int G) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int na = S.misc[0];
  if (P.mfma) {
    // Workgroups are dealt to the XCDs in turn (wg % 8 on XCD wg % 8), each
    // XCD with its own L2.  Each list is cut into one chunk of equal modelled
    // work per XCD, and a chunk's units are dealt to the XCD's workgroups in
    // turn (workgroup j of the XCD takes units j, j + per, ...): at any time
    // the XCD's workgroups work on the units of two or three experts, whose
    // activation tiles (x of the experts' tokens, h) then stay in its L2
    // instead of being fetched again for each unit (measured at T=512 with
    // contiguous per-workgroup ranges: 32 experts' x per XCD, twice the L2).
    const int nx = (G % 8 == 0 && G >= 16) ? 8 : 1;
    const int per = G / nx, xcd = wg % nx, j = wg / nx;
    const int Rg = (P.F + kGUUnitRows - 1) / kGUUnitRows;
    if (wave < 4) {  // waves 0-3: gate/up chunk start and end, down chunk start and end
      const bool gu = wave < 2;
      const int R = gu ? Rg : (P.d + kDnUnitRows - 1) / kDnUnitRows;
      const int v = row_at(gu ? S.cgu : S.cdn, na, R, xcd + (wave & 1), nx);
      if (lane == 0) S.misc[wave == 0 ? 5 : wave == 1 ? 3 : wave == 2 ? 6 : 4] = v;
    }
    __syncthreads();
    if (wave == 0) {
      const int pos = per <= kWave ? order_down(S, per, j, Rg) : j;
      if (lane == 0) {
        S.misc[5] += j;
        S.misc[6] += pos;
        S.misc[kMiscStride] = per;
      }
    }
    __syncthreads();
    return;
  }
  // The gate/up chunk boundaries b = 2k + side of chunk k (side 0 its start,
  // 1 its end), two per wave; waves 4 and 5 also the two down chunks'
  // boundaries (the searches of one wave run one after another: four per
  // wave on waves 0-3 took ~1 us more before the first weight loads)
  {
    int* tab = round_tab(S, 0);
    const int nr = P.xmode ? 1 : kRounds;  // xmode 1: one range (its pairs' x is staged)
    for (int b = wave; b < 2 * nr; b += kWaves) {
      const int k = b >> 1, side = b & 1;
      const int v = row_at(S.cgu, na, P.F, k * G + wg + side, nr * G);
      if (lane == 0) tab[side ? kRounds + k : k] = v;  // ends parked where the lengths go
    }
    if (wave == 0 && lane == 0)
      for (int c = nr; c < kRounds; ++c) tab[c] = tab[kRounds + c] = 0;  // empty chunks
  }
  if (wave == 4 || wave == 5) {
    int* tab = round_tab(S, 1);
    const int side = wave & 1;
    const int v = row_at(S.cdn, na, P.d / kDnRows, wg + side, G);
    if (lane == 0) {
      tab[side ? kRounds : 0] = v;
      if (wave == 4)
        for (int c = 1; c < kRounds; ++c) tab[c] = tab[kRounds + c] = 0;  // empty chunks
    }
  }
  __syncthreads();
  // chunk lengths -> cumulative starts, both tables at once by wave 0: lanes
  // 0-7 (gate/up) and 32-39 (down) hold a chunk's length; exclusive sums
  // within each group of 32 lanes by the wave scan (the upper group's scan
  // starts from the lower group's total, which is subtracted)
  if (wave == 0) {
    const int ph = lane >> 5, k = lane & 31;
    int* t = round_tab(S, ph);
    const int len = k < kRounds ? t[kRounds + k] - t[k] : 0;
    const int inc = wave_inclusive_scan(len);
    const int base = __shfl(inc, 31);  // the lower group's total
    const int incl = ph ? inc - base : inc;
    if (k < kRounds) t[kRounds + k] = incl - len;
    if (k == kRounds - 1) t[2 * kRounds] = incl;
    if (k == 0) S.misc[1 + ph] = 0;
  }
  __syncthreads();
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its outstanding global loads (HIP's __syncthreads also
// waits for every global load in flight, which would drain the weight
// prefetch at every K block).
__device__ __forceinline__ void lds_barrier() {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ------------------------------------ large batches: MFMA expert steps -----
// When x does not fit in LDS the expert GEMMs run on v_mfma_f32_16x16x32_bf16:
// A = weights decoded exactly to bf16 (E2M1 * 2^k is a bf16), B = activations
// as bf16: x exactly, h as hi + lo bf16 (two MFMAs, ~16 significant bits).
// A workgroup unit covers 8 wave tiles of rows of one expert; its waves walk
// the K blocks of 128 in lockstep, and the activation tile of each K block
// (all of the unit's tokens in this pass) is staged once in LDS for all of
// them.  A K block is one 16-byte code chunk per lane: lane l holds row
// l % 16, chunk 4j + l / 16, i.e. K elements 128j + 32(l/16) .. +32; MFMA
// step s uses elements 8s .. 8s+7 of it, and B supplies the same K elements
// (128j + 32(l/16) + 8s .. +8) for column l % 16, so each MFMA sums a
// permuted but matching set of 32 K indices.

// Position in a workgroup's stream of (unit, token pass, K block).
struct Seg {
  int k, u, pass, j;  // index in the workgroup's list, unit, first token of the pass, K block
  int e, p0, ne;    // expert, its first pair, its tokens
  bool valid;
};

__device__ __forceinline__ void seg_unit(const Smem& S, int u, int R, Seg& c) {
  c.u = u;
  c.pass = 0;
  c.j = 0;
  c.e = uni(S.act[u / R]);
  c.p0 = uni(S.off[c.e]);
  c.ne = uni(S.off[c.e + 1]) - c.p0;
}

// Unit k of the workgroup's units of step ph (0 gate/up, 1 down), or -1 past
// its end (see set_ranges).
__device__ __forceinline__ int wg_unit(const Smem& S, int ph, int k) {
  const int u = uni(S.misc[ph ? 6 : 5]) + k * uni(S.misc[kMiscStride]);
  return u < uni(S.misc[ph ? 4 : 3]) ? u : -1;
}

__device__ __forceinline__ void seg_start(const Smem& S, int ph, int R, Seg& c) {
  c.k = 0;
  const int u = wg_unit(S, ph, 0);
  c.valid = u >= 0;
  if (c.valid) seg_unit(S, u, R, c);
}

__device__ __forceinline__ void seg_next(const Smem& S, int ph, int R, int nkb, int pass_len, Seg& c) {
  if (!c.valid) return;
  if (++c.j < nkb) return;
  c.j = 0;
  c.pass += pass_len;
  if (c.pass < c.ne) return;
  const int u = wg_unit(S, ph, ++c.k);
  if (u >= 0) seg_unit(S, u, R, c);
  else c.valid = false;
}

// Number of positions (unit, pass, K block) in the workgroup's list of step ph.
__device__ __forceinline__ int seg_count(const Smem& S, int ph, int R, int nkb, int pass_len) {
  int n = 0;
  for (int k = 0;; ++k) {
    const int u = wg_unit(S, ph, k);
    if (u < 0) break;
    const int e = uni(S.act[u / R]);
    const int ne = uni(S.off[e + 1]) - uni(S.off[e]);
    n += (ne + pass_len - 1) / pass_len;
  }
  return n * nkb;
}

// ---- gate/up ----
// Both expert steps move through their stream one step at a time: the x (or
// h) tile of the next step is loaded first, then the next step's weights, then
// the current step is computed from registers and LDS, then the next tile is
// written to LDS and the workgroup synchronises.  Waiting for the next tile
// therefore never waits for the next step's weights (loads complete in issue
// order), and each wave keeps 8 KiB of weights in flight while it computes.

// ---- gate/up ----
struct GUA {
  u32x4_t g[kGUK], u[kGUK];
  uint32_t sg[kGUK], su[kGUK];  // scale bytes as loaded (byte loads)
  u32x4_t sv;                   // wide scale loads: lane l < 16 row l of W_gate, 16 <= l < 32 row l - 16 of W_up
  uint32_t keep;                // bit b: K block b's chunk is in range
};

// This wave's tile of step c: rows r0 .. r0 + 15 (r0 = (u % R) * 128 + 16 *
// wave) of W_gate and W_up, chunks 16 j .. 16 j + 15 (kGUK = 4 K blocks of 4
// chunks).  The loads read whole 128-byte lines: load i takes rows
// r0 + 8 (i & 1) + (l / 4) % 8, chunks 16 j + 8 (i >> 1) + 4 (l / 32) + l % 4
// (four lanes per 64-byte half of a row, lanes 0-31 the first halves).  The
// MFMA layout wants lane l to hold row r0 + l % 16, chunk
// 16 j + 4 b + l / 16 for K block b, i.e. four 64-byte pieces per row spread
// over four loads; loads of that shape moved the same bytes in half-lines and
// made the T=512 layer 25% slower (2.58 instead of 2.07 ms).  gu_mfma_take
// moves the data into the MFMA layout when it is used.  Rows past F (last
// unit of an expert) and chunks past d read a valid chunk and get a zero scale
// at use.  Nothing is computed from the loaded data here, so the loads stay in
// flight.  WS (d a multiple of 512, so a row's 16 scale bytes of a step are
// 16-byte aligned): the scales of the step come in one 16-byte load per row
// (lanes 0-15 W_gate, 16-31 W_up) instead of one byte load per lane per K
// block and matrix, 1 load instruction instead of 8 (the loads' address
// processing is one of the step's limits, see gu_mfma_take).
template <bool WS>
__device__ __forceinline__ void gu_mfma_load(const Params& P, const Seg& c, int R, GUA& A) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int d = P.d, F = P.F, NCH = d / 32;
  const int r0 = (c.u % R) * kGUUnitRows + 16 * wave;
  // one expert's codes and scales through buffer descriptors: 32-bit offsets
  // (an expert is at most 3 * 8192 * 4096 / 2 bytes)
  const uint32_t pbytes = (uint32_t)(3 * d / 2) * (uint32_t)F, sbytes = (uint32_t)(3 * NCH) * (uint32_t)F;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(P.packed + (size_t)c.e * pbytes, pbytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(P.scales + (size_t)c.e * sbytes, sbytes);
  const uint32_t up = (uint32_t)F * (uint32_t)(d / 2), sup = (uint32_t)F * (uint32_t)NCH;
  A.keep = 0;
#pragma unroll
  for (int i = 0; i < kGUK; ++i) {
    const int rr = min(r0 + 8 * (i & 1) + ((lane >> 2) & 7), F - 1);
    const int cc = min(16 * c.j + 8 * (i >> 1) + 4 * (lane >> 5) + (lane & 3), NCH - 1);
    const uint32_t po = (uint32_t)rr * (uint32_t)(d / 2) + (uint32_t)cc * 16u;
    const uint32_t so = (uint32_t)rr * (uint32_t)NCH + (uint32_t)cc;
    A.g[i] = ld_stream16_buf(pr, po);
    A.u[i] = ld_stream16_buf(pr, po + up);
    if (!WS) {
      A.sg[i] = ld_byte_buf(sr, so);
      A.su[i] = ld_byte_buf(sr, so + sup);
    }
    // in range, for the MFMA-layout chunk this lane will hold for block i
    const int row = r0 + (lane & 15), ch = 16 * c.j + 4 * i + (lane >> 4);
    A.keep |= (row < F && ch < NCH) ? 1u << i : 0u;
  }
  if (WS) {
    // bytes past the row's chunks (last step) belong to other rows or read
    // past the descriptor (zeros); their chunks are out of range (keep).
    // Through the L2 without the streaming hint: a 128-byte line of scales
    // serves 8 steps of its row (streaming loads fetched it again for each:
    // 1.3x the layer's HBM bytes at T=128 and T=512)
    const uint32_t so = (uint32_t)min(r0 + (lane & 15), F - 1) * (uint32_t)NCH + 16u * (uint32_t)c.j;
    A.sv = ld_cached16(sr, lane < 32 ? so + (lane >= 16 ? sup : 0u) : 0xFFFFFFF0u);
  }
}
// K block b of the MFMA layout from the loads: lane l = 16 h + r takes chunk
// 4 b + h of row r, held by load 2 (b >> 1) + (r >> 3) of lane
// 32 (b & 1) + 4 (r & 7) + h: every permute reads one half of the wave.  With
// eight lanes per whole line (sources 8 (r & 7) + 4 (b & 1) + h, in both
// halves) the sources s and s + 32 shared an LDS bank, and the layer was ~1%
// slower at T=128 and T=512.  Orders with rows varying fastest across the
// lanes (11% slower gate/up step at T=512) or the chunks of a line rotated by
// the row (2% slower) avoid the conflicts too but break the loads' runs of
// consecutive bytes, which their address processing needs.
__device__ __forceinline__ uint32_t bperm(uint32_t v, int addr) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v);
}
template <bool WS>
__device__ __forceinline__ void gu_mfma_take(const GUA& A, int b, u32x4_t& g, u32x4_t& u, uint32_t& sg,
                                             uint32_t& su) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, h = lane >> 4;
  const int addr = 4 * (32 * (b & 1) + 4 * (r & 7) + h);
  const bool hi = r >= 8;
  const int i0 = 2 * (b >> 1), i1 = i0 + 1;
  const auto pick = [&](uint32_t a0, uint32_t a1) {
    const uint32_t v0 = bperm(a0, addr), v1 = bperm(a1, addr);
    return hi ? v1 : v0;
  };
  g.x = pick(A.g[i0].x, A.g[i1].x);
  g.y = pick(A.g[i0].y, A.g[i1].y);
  g.z = pick(A.g[i0].z, A.g[i1].z);
  g.w = pick(A.g[i0].w, A.g[i1].w);
  u.x = pick(A.u[i0].x, A.u[i1].x);
  u.y = pick(A.u[i0].y, A.u[i1].y);
  u.z = pick(A.u[i0].z, A.u[i1].z);
  u.w = pick(A.u[i0].w, A.u[i1].w);
  if (WS) {
    // chunk 16 j + 4 b + h of row r: byte h of dword b of lane r (W_gate) or
    // lane 16 + r (W_up)
    const uint32_t d = b == 0 ? A.sv.x : b == 1 ? A.sv.y : b == 2 ? A.sv.z : A.sv.w;
    sg = (bperm(d, 4 * r) >> (8 * h)) & 0xFFu;
    su = (bperm(d, 4 * (16 + r)) >> (8 * h)) & 0xFFu;
  } else {
    sg = pick(A.sg[i0], A.sg[i1]);
    su = pick(A.su[i0], A.su[i1]);
  }
}

// x tile of step c: token rows n < 32 of the pass, K blocks kGUK j .. +kGUK,
// four 16-byte pieces per thread; LDS layout [block][token][272 bytes].
// `ok` bit m marks pieces that hold data (others are written as zeros).
constexpr int kXPieces = kGUK * kGUPass * 16 / kWG;
static_assert(kGUK == 4 && kXPieces == 4, "piece index = token(5) | block(2) | piece(4) bits");
// Token rows of the x tile pieces a thread loads: piece m of thread i is
// token n = i / 64 + 8 m of the pass (the same for the whole wave), K element
// 128 b + 8 q of the step's 512 (b = (i / 16) % 4, q = i % 16).  The rows
// (token * d) change only with the pass, so they are looked up once per pass
// (key: the pass's first pair).
struct XRows {
  int key;
  int row[kXPieces];
};
__device__ __forceinline__ void gu_mfma_xload(const Params& P, const Smem& S, const Seg& c, XRows& xr,
                                              u32x4_t (&v)[kXPieces], uint32_t& ok) {
  const int TK = P.T * P.k;
  const int np = min(kGUPass, c.ne - c.pass);
  const int wave = threadIdx.x / kWave;
  const __amdgpu_buffer_rsrc_t xd = make_rsrc(P.x, (uint32_t)((size_t)P.T * P.d * 2));
  const int key = c.p0 + c.pass;
  if (c.valid && key != xr.key) {  // uniform
    xr.key = key;
#pragma unroll
    for (int m = 0; m < kXPieces; ++m)
      xr.row[m] = uni(S.slot[min(key + wave + 8 * m, TK - 1)] / P.k) * P.d;
  }
  const int kk = c.j * (kGUK * kKB) + (((int)threadIdx.x >> 4) & 3) * kKB + 8 * ((int)threadIdx.x & 15);
  ok = 0;
#pragma unroll
  for (int m = 0; m < kXPieces; ++m) {
    const bool use = c.valid && wave + 8 * m < np && kk < P.d;
    // pieces past the pass's tokens or past d read past the descriptor's
    // end: no memory access, zeros (and they are written as zeros)
    const uint32_t off = use ? (uint32_t)(xr.row[m] + kk) * 2u : 0xFFFFFFF0u;
    v[m] = ld_cached16(xd, off);
    ok |= use ? 1u << m : 0u;
  }
}

__device__ __forceinline__ void gu_mfma_xstore(char* tile, const u32x4_t (&v)[kXPieces], uint32_t ok) {
#pragma unroll
  for (int m = 0; m < kXPieces; ++m) {
    const int pc = (int)threadIdx.x + kWG * m;
    const int n = pc >> 6, b = (pc >> 4) & 3, q = pc & 15;
    *reinterpret_cast<u32x4_t*>(tile + (b * kGUPass + n) * kTileRow + q * 16) =
        (ok >> m) & 1u ? v[m] : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// MFMAs of one step for this wave's tile against the x tile in LDS, for the
// first NG column groups of 16 tokens.
template <int NG, bool WS>
__device__ __forceinline__ void gu_mfma_step(const GUA& A, const char* tile, f32x4_t (&ag)[2], f32x4_t (&au)[2]) {
  const int lane = threadIdx.x & (kWave - 1);
  const char* b0 = tile + (lane & 15) * kTileRow + (lane >> 4) * 64;
#pragma unroll
  for (int b = 0; b < kGUK; ++b) {
    bf16x8_t x[4][NG];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        x[s][g] = *reinterpret_cast<const bf16x8_t*>(b0 + (b * kGUPass + g * 16) * kTileRow + s * 16);
    const bool in = (A.keep >> b) & 1u;
    u32x4_t cg, cu;
    uint32_t sgb, sub;
    gu_mfma_take<WS>(A, b, cg, cu, sgb, sub);
    bf16x8_t wg[4], wu[4];
    decode_chunk_a(cg, e8m0_to_f32(in ? sgb : 0u), wg);
    decode_chunk_a(cu, e8m0_to_f32(in ? sub : 0u), wu);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        ag[g] = mfma_bf16(wg[s], x[s][g], ag[g]);
        au[g] = mfma_bf16(wu[s], x[s][g], au[g]);
      }
    }
  }
}

// h = silu(g) * u of this wave's tile for the pass's tokens, as tagged words.
__device__ __forceinline__ void gu_mfma_store(const Params& P, const Seg& c, int R, uint32_t tag, f32x4_t (&ag)[2],
                                              f32x4_t (&au)[2]) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int np = min(kGUPass, c.ne - c.pass);
  const int row0 = (c.u % R) * kGUUnitRows + 16 * wave;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(P.hq, (uint32_t)((size_t)P.T * P.k * P.F * 8));
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int n = 16 * g + (lane & 15);
    if (row0 < P.F && n < np) {
      const size_t w0 = (size_t)(c.p0 + c.pass + n) * P.F + row0 + 4 * (lane >> 4);
      uint32_t hb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hb[i] = __builtin_bit_cast(uint32_t, swiglu(ag[g][i], au[g][i]));
      if (P.narrow) {  // uniform
        st_tagged2(rs, (uint32_t)(w0 * 8), hb[0], hb[1], tag);
        st_tagged2(rs, (uint32_t)(w0 * 8 + 16), hb[2], hb[3], tag);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) st_tagged(P.hq + w0 + i, hb[i], tag);
      }
    }
    ag[g] = au[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// One step q: prefetch the x tile of step q + 1 into registers (n1) and the
// weights of step q + 2 (n2, into An2), compute step q (weights Ac, LDS tile
// `cur`), write tile q + 1 into LDS tile `nxt`, synchronise.  The weights are
// in flight for two steps: with one step, a step's loads were waited for at
// the next step (a step's compute and the x tile take less than one loaded
// memory latency).
template <bool WS>
__device__ __forceinline__ void gu_mfma_one(const Params& P, const Smem& S, uint32_t tag, int R, int nst,
                                            int q, int npos, Seg& cc, Seg& n1, Seg& n2, XRows& xrows, const GUA& Ac,
                                            GUA& An2, char* cur, char* nxt, f32x4_t (&ag)[2], f32x4_t (&au)[2]) {
  u32x4_t xv[kXPieces];
  uint32_t xok;
  gu_mfma_xload(P, S, n1, xrows, xv, xok);  // first: waiting for it below must not wait for An2
  gu_mfma_load<WS>(P, n2, R, An2);
  if (cc.ne - cc.pass > 16)
    gu_mfma_step<2, WS>(Ac, cur, ag, au);
  else
    gu_mfma_step<1, WS>(Ac, cur, ag, au);
  if (cc.j == nst - 1) gu_mfma_store(P, cc, R, tag, ag, au);
  if (q + 1 < npos) gu_mfma_xstore(nxt, xv, xok);
  seg_next(S, 0, R, nst, kGUPass, cc);
  seg_next(S, 0, R, nst, kGUPass, n1);
  seg_next(S, 0, R, nst, kGUPass, n2);
  lds_barrier();
}

// Gate/up + SwiGLU for the workgroup's units [U0, U1) (equal shares of the
// modelled work).  All threads of the workgroup.  Three weight buffers
// (steps q, q + 1, q + 2), two LDS x tiles.
template <bool WS>
__device__ __forceinline__ void gate_up_mfma_ws(const Params& P, const Smem& S, uint32_t tag, int wg, int G) {
  const int R = (P.F + kGUUnitRows - 1) / kGUUnitRows;
  const int nst = (P.d + kGUK * kKB - 1) / (kGUK * kKB);
  const int npos = seg_count(S, 0, R, nst, kGUPass);
  if (npos == 0) return;
  char* cur = reinterpret_cast<char*>(S.xs);
  char* nxt = cur + kGUK * kGUPass * kTileRow;
  Seg cc, n1, n2;
  seg_start(S, 0, R, cc);
  n1 = cc;
  seg_next(S, 0, R, nst, kGUPass, n1);
  n2 = n1;
  seg_next(S, 0, R, nst, kGUPass, n2);
  GUA A0, A1, A2;
  f32x4_t ag[2], au[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) ag[g] = au[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  XRows xrows;
  xrows.key = -1;
  {
    u32x4_t xv[kXPieces];
    uint32_t xok;
    gu_mfma_xload(P, S, cc, xrows, xv, xok);
    gu_mfma_load<WS>(P, cc, R, A0);
    gu_mfma_load<WS>(P, n1, R, A1);
    gu_mfma_xstore(cur, xv, xok);
    lds_barrier();
  }
  const auto swap_tiles = [&] {
    char* t = cur;
    cur = nxt;
    nxt = t;
  };
  for (int q = 0; q < npos; q += 3) {
    gu_mfma_one<WS>(P, S, tag, R, nst, q, npos, cc, n1, n2, xrows, A0, A2, cur, nxt, ag, au);
    if (q + 1 >= npos) break;
    swap_tiles();
    gu_mfma_one<WS>(P, S, tag, R, nst, q + 1, npos, cc, n1, n2, xrows, A1, A0, cur, nxt, ag, au);
    if (q + 2 >= npos) break;
    swap_tiles();
    gu_mfma_one<WS>(P, S, tag, R, nst, q + 2, npos, cc, n1, n2, xrows, A2, A1, cur, nxt, ag, au);
    swap_tiles();
  }
}
__device__ __forceinline__ void gate_up_mfma(const Params& P, const Smem& S, uint32_t tag, int wg, int G) {
  if (P.d % 512 == 0)  // uniform
    gate_up_mfma_ws<true>(P, S, tag, wg, G);
  else
    gate_up_mfma_ws<false>(P, S, tag, wg, G);
}

// ---- down ----
struct DnA {
  u32x4_t w[kDnK * kDnTiles];  // as loaded (load i)
  uint32_t s[kDnK * kDnTiles]; // scale bytes as loaded (byte loads)
  u32x2_t sv;                  // wide scale loads: lane l the step's 8 scale bytes of row r0 + l
  uint32_t keep;               // bit b * kDnTiles + t: the MFMA-layout chunk of tile t, block b is in range
};
static_assert(kDnK == 2, "a step covers one 128-byte line (8 chunks) of each W_down row");

// This wave's 4 tiles of step c: rows r0 .. r0 + 63 (r0 = (u % R) * 512 +
// 64 * wave) of W_down, chunks 8 j .. 8 j + 7 (K = F): one 128-byte line per
// row.  Load i takes rows r0 + 8 i + l / 8, chunk 8 j + l % 8 (whole lines; see
// gu_mfma_load); dn_mfma_take moves tile t, block b into the MFMA layout
// (lane l: row r0 + 16 t + l % 16, chunk 8 j + 4 b + l / 16).  WS (ffn a
// multiple of 256): the step's 8 scale bytes of row r0 + l in one 8-byte load
// by lane l, 1 load instruction instead of 8 byte loads.
template <bool WS>
__device__ __forceinline__ void dn_mfma_load(const Params& P, const Seg& c, int R, DnA& A) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int d = P.d, F = P.F, NCH = F / 32;
  // W_down of one expert through buffer descriptors (32-bit offsets)
  const uint32_t pbytes = (uint32_t)(3 * d / 2) * (uint32_t)F, sbytes = (uint32_t)(3 * d / 32) * (uint32_t)F;
  const uint32_t dn = (uint32_t)F * (uint32_t)d;  // W_down after W_gate and W_up
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(P.packed + (size_t)c.e * pbytes + dn, dn / 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(P.scales + (size_t)c.e * sbytes + dn / 16, dn / 32);
  const int r0 = (c.u % R) * kDnUnitRows + 64 * wave;
  const int cc = min(8 * c.j + (lane & 7), NCH - 1);
  A.keep = 0;
#pragma unroll
  for (int i = 0; i < kDnK * kDnTiles; ++i) {
    const int rr = min(r0 + 8 * i + (lane >> 3), d - 1);
    A.w[i] = ld_stream16_buf(pr, (uint32_t)rr * (uint32_t)(F / 2) + (uint32_t)cc * 16u);
    if (!WS) A.s[i] = ld_byte_buf(sr, (uint32_t)rr * (uint32_t)NCH + (uint32_t)cc);
  }
  // (through the L2: a 128-byte line of scales serves 16 steps of its row)
  if (WS) A.sv = ld_cached8_buf(sr, (uint32_t)min(r0 + lane, d - 1) * (uint32_t)NCH + 8u * (uint32_t)c.j);
#pragma unroll
  for (int b = 0; b < kDnK; ++b)
#pragma unroll
    for (int t = 0; t < kDnTiles; ++t) {
      const int row = r0 + 16 * t + (lane & 15), ch = 8 * c.j + 4 * b + (lane >> 4);
      A.keep |= (row < d && ch < NCH) ? 1u << (b * kDnTiles + t) : 0u;
    }
}
// Tile t, block b in the MFMA layout: lane l = 16 h + r takes row 16 t + r,
// chunk 4 b + h, held by load 2 t + (r >> 3) of lane 8 (r & 7) + 4 b + h.
template <bool WS>
__device__ __forceinline__ void dn_mfma_take(const DnA& A, int b, int t, u32x4_t& w, uint32_t& sc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, h = lane >> 4;
  const int addr = 4 * (8 * (r & 7) + 4 * b + h);
  const bool hi = r >= 8;
  const int i0 = 2 * t, i1 = i0 + 1;
  const auto pick = [&](uint32_t a0, uint32_t a1) {
    const uint32_t v0 = bperm(a0, addr), v1 = bperm(a1, addr);
    return hi ? v1 : v0;
  };
  w.x = pick(A.w[i0].x, A.w[i1].x);
  w.y = pick(A.w[i0].y, A.w[i1].y);
  w.z = pick(A.w[i0].z, A.w[i1].z);
  w.w = pick(A.w[i0].w, A.w[i1].w);
  if (WS)  // chunk 8 j + 4 b + h of row 16 t + r: byte h of dword b of lane 16 t + r
    sc = (bperm(b == 0 ? A.sv.x : A.sv.y, 4 * (16 * t + r)) >> (8 * h)) & 0xFFu;
  else
    sc = pick(A.s[i0], A.s[i1]);
}

// h tile of step c: pairs n < 32 of the pass, values 128(kDnK j) .. +128 kDnK
// as tagged words, 16-byte coherent loads of two words (row n = piece /
// kHRow, word pair = piece % kHRow).
constexpr int kHRow = kDnK * kKB / 2;  // word pairs per pair row of a step
constexpr int kHPieces = kDnPass * kHRow / kWG;
// NR: the pass has at most NR pairs (16 or 32): only the pieces of its first
// NR rows are loaded and written (a tile of at most 16 pairs feeds only the
// first column group, so rows 16-31 are never read: 4 of the 8 loads per
// thread per step saved, the loads' address processing being one of the
// step's limits).
template <bool COHERENT, int NR>
__device__ __forceinline__ void dn_mfma_hload(const Params& P, const Seg& c, __amdgpu_buffer_rsrc_t rs,
                                              u32x4_t (&v)[kHPieces]) {
  static_assert(NR % (kWG / kHRow) == 0 && NR <= kDnPass, "whole pieces");
  const int np = min(kDnPass, c.ne - c.pass);
#pragma unroll
  for (int m = 0; m < NR / (kWG / kHRow); ++m) {
    const int pc = (int)threadIdx.x + kWG * m;
    const int n = pc / kHRow, k = c.j * kDnK * kKB + 2 * (pc % kHRow);
    // pieces past the pass's pairs or past F read past the descriptor's end:
    // no memory access, zeros (dn_mfma_hstore neither checks nor uses them)
    const bool use = c.valid && n < np && k < P.F;
    const uint32_t off = use ? ((uint32_t)(c.p0 + c.pass + n) * (uint32_t)P.F + (uint32_t)k) * 8u : 0xFFFFFFF0u;
    v[m] = COHERENT ? ld_coherent16(rs, off) : ld_cached16(rs, off);
  }
}

// Checks the tags of a staged h tile (re-reading it until they are current;
// after a watchdog abort it gives up and sets *bad, an LDS flag after which
// the workgroup stores no more results), then writes it
// as bf16 hi and lo tiles, layout [block][pair][272 bytes] each.  Values past
// the pass or past F are zero.
template <int NR>
__device__ __forceinline__ void dn_mfma_hstore(const Params& P, const Seg& c, __amdgpu_buffer_rsrc_t rs,
                                               uint32_t tag, u32x4_t (&v)[kHPieces], char* hi_tile,
                                               char* lo_tile, int* bad) {
  constexpr int kM = NR / (kWG / kHRow);  // pieces of the first NR rows
  const int np = min(kDnPass, c.ne - c.pass);
  auto used = [&](int m) {
    const int pc = (int)threadIdx.x + kWG * m;
    return c.valid && pc / kHRow < np && c.j * kDnK * kKB + 2 * (pc % kHRow) < P.F;
  };
  auto current = [&]() {
    bool ok = true;
#pragma unroll
    for (int m = 0; m < kM; ++m) ok &= !used(m) || (v[m].y == tag + P.withhold_h && v[m].w == tag + P.withhold_h);
    return ok;
  };
  if (!__all(current())) {
    const uint64_t t0 = wall_clock64();
    int round = 0;
    for (;;) {
      if (!keep_waiting(P, tag, t0, kSiteH, c.p0 + c.pass, round, 3)) {
        // the tile is written anyway (every wave keeps to the workgroup's
        // barriers), but no result computed from it is stored
        *bad = 1;
        break;
      }
      dn_mfma_hload<true, NR>(P, c, rs, v);
      if (__all(current())) break;
    }
  }
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const int pc = (int)threadIdx.x + kWG * m;
    const int n = pc / kHRow, w = pc % kHRow;  // w: word pair within the step's values
    const int off = ((w >> 6) * kDnPass + n) * kTileRow + (w & 63) * 4;
    const bool u = used(m);
    __bf16 h0, l0, h1, l1;
    split_bf16(u ? u2f(v[m].x) : 0.f, h0, l0);
    split_bf16(u ? u2f(v[m].z) : 0.f, h1, l1);
    *reinterpret_cast<bf16x2_t*>(hi_tile + off) = bf16x2_t{h0, h1};
    *reinterpret_cast<bf16x2_t*>(lo_tile + off) = bf16x2_t{l0, l1};
  }
}

// Operand s of a decoded chunk (elements 8s .. 8s+7, times the scale).
__device__ __forceinline__ bf16x8_t decode_op_a(const u32x4_t w, float scale, int s) {
  const uint32_t ws = s == 0 ? w.x : s == 1 ? w.y : s == 2 ? w.z : w.w;
  const bf16x2_t p0 = fp4x2_to_bf16x2<0>(ws, scale), p1 = fp4x2_to_bf16x2<1>(ws, scale);
  const bf16x2_t p2 = fp4x2_to_bf16x2<2>(ws, scale), p3 = fp4x2_to_bf16x2<3>(ws, scale);
  return bf16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

template <int NG, bool WS>
__device__ __forceinline__ void dn_mfma_step(const DnA& A, const char* hi_tile, const char* lo_tile,
                                             f32x4_t (&acc)[kDnTiles][2]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int boff = (lane & 15) * kTileRow + (lane >> 4) * 64;
#pragma unroll
  for (int b = 0; b < kDnK; ++b) {
    float sc[kDnTiles];
    u32x4_t wt[kDnTiles];
#pragma unroll
    for (int t = 0; t < kDnTiles; ++t) {
      uint32_t sb;
      dn_mfma_take<WS>(A, b, t, wt[t], sb);
      sc[t] = e8m0_to_f32((A.keep >> (b * kDnTiles + t)) & 1u ? sb : 0u);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t bh[NG], bl[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int o = boff + (b * kDnPass + g * 16) * kTileRow + s * 16;
        bh[g] = *reinterpret_cast<const bf16x8_t*>(hi_tile + o);
        bl[g] = *reinterpret_cast<const bf16x8_t*>(lo_tile + o);
      }
      bf16x8_t a[kDnTiles];
#pragma unroll
      for (int t = 0; t < kDnTiles; ++t) a[t] = decode_op_a(wt[t], sc[t], s);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int t = 0; t < kDnTiles; ++t) {
          acc[t][g] = mfma_bf16(a[t], bh[g], acc[t][g]);
          acc[t][g] = mfma_bf16(a[t], bl[g], acc[t][g]);
        }
      }
    }
  }
}

// gate * y of this wave's 4 tiles for the pass's tokens, as tagged words in
// the tokens' slot rows.
__device__ __forceinline__ void dn_mfma_store(const Params& P, const Smem& S, const Seg& c, int R, uint32_t tag,
                                              f32x4_t (&acc)[kDnTiles][2]) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int np = min(kDnPass, c.ne - c.pass);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(P.yq, (uint32_t)((size_t)P.T * P.k * P.d * 8));
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int n = 16 * g + (lane & 15);
    const int slot = n < np ? S.slot[min(c.p0 + c.pass + n, P.T * P.k - 1)] : 0;
    const float gate = n < np ? S.tkw[slot] : 0.f;
#pragma unroll
    for (int t = 0; t < kDnTiles; ++t) {
      const int row0 = (c.u % R) * kDnUnitRows + 64 * wave + 16 * t;
      if (row0 < P.d && n < np) {
        const size_t w0 = (size_t)slot * P.d + row0 + 4 * (lane >> 4);
        uint32_t yb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) yb[i] = __builtin_bit_cast(uint32_t, gate * acc[t][g][i]);
        if (P.narrow) {  // uniform
          st_tagged2(rs, (uint32_t)(w0 * 8), yb[0], yb[1], tag);
          st_tagged2(rs, (uint32_t)(w0 * 8 + 16), yb[2], yb[3], tag);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) st_tagged(P.yq + w0 + i, yb[i], tag);
        }
      }
      acc[t][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
}

template <bool WS, int NR>
__device__ __forceinline__ void dn_mfma_one_nr(const Params& P, const Smem& S, uint32_t tag, int R, int nst,
                                               int q, int npos, __amdgpu_buffer_rsrc_t rs, Seg& cc, Seg& nc,
                                               const DnA& Ac, DnA& An, char* cur, char* nxt,
                                               f32x4_t (&acc)[kDnTiles][2], int* bad) {
  constexpr int kHalf = kDnK * kDnPass * kTileRow;  // hi tile; lo tile follows
  // read after the barrier that ended the previous step: set if any tile up to
  // the current one failed its wait (the flag never clears within a call)
  const bool ok = *bad == 0;
  u32x4_t hr[kHPieces];
  dn_mfma_hload<false, NR>(P, nc, rs, hr);  // first: waiting for it below must not wait for An
  dn_mfma_load<WS>(P, nc, R, An);
  if (cc.ne - cc.pass > 16)
    dn_mfma_step<2, WS>(Ac, cur, cur + kHalf, acc);
  else
    dn_mfma_step<1, WS>(Ac, cur, cur + kHalf, acc);
  if (cc.j == nst - 1 && ok) dn_mfma_store(P, S, cc, R, tag, acc);
  if (q + 1 < npos) dn_mfma_hstore<NR>(P, nc, rs, tag, hr, nxt, nxt + kHalf, bad);
  seg_next(S, 1, R, nst, kDnPass, cc);
  seg_next(S, 1, R, nst, kDnPass, nc);
  lds_barrier();
}
// The next tile (nc) decides which h pieces are loaded (dn_mfma_hload).
template <bool WS>
__device__ __forceinline__ void dn_mfma_one(const Params& P, const Smem& S, uint32_t tag, int R, int nst,
                                            int q, int npos, __amdgpu_buffer_rsrc_t rs, Seg& cc, Seg& nc,
                                            const DnA& Ac, DnA& An, char* cur, char* nxt,
                                            f32x4_t (&acc)[kDnTiles][2], int* bad) {
  if (nc.ne - nc.pass <= 16)  // uniform (an invalid nc loads nothing either way)
    dn_mfma_one_nr<WS, 16>(P, S, tag, R, nst, q, npos, rs, cc, nc, Ac, An, cur, nxt, acc, bad);
  else
    dn_mfma_one_nr<WS, kDnPass>(P, S, tag, R, nst, q, npos, rs, cc, nc, Ac, An, cur, nxt, acc, bad);
}

// Down projection for the workgroup's units [U0, U1).  All threads.  False
// if an h wait was abandoned (then some of the units' results are not stored).
template <bool WS>
__device__ __forceinline__ bool down_mfma_ws(const Params& P, const Smem& S, uint32_t tag, int wg, int G) {
  __shared__ int s_bad;
  const int R = (P.d + kDnUnitRows - 1) / kDnUnitRows;
  const int nst = (P.F + kDnK * kKB - 1) / (kDnK * kKB);
  const int npos = seg_count(S, 1, R, nst, kDnPass);
  if (npos == 0) return true;
  if (threadIdx.x == 0) s_bad = 0;
  lds_barrier();  // before any wave can set it
  constexpr int kHalf = kDnK * kDnPass * kTileRow;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(P.hq, (uint32_t)((size_t)P.T * P.k * P.F * 8));
  char* t0 = reinterpret_cast<char*>(S.xs);
  char* t1 = t0 + 2 * kHalf;
  Seg cc, nc;
  seg_start(S, 1, R, cc);
  nc = cc;
  DnA A0, A1;
  f32x4_t acc[kDnTiles][2];
#pragma unroll
  for (int t = 0; t < kDnTiles; ++t) acc[t][0] = acc[t][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  {
    u32x4_t hr[kHPieces];
    dn_mfma_hload<false, kDnPass>(P, nc, rs, hr);
    dn_mfma_load<WS>(P, nc, R, A0);
    dn_mfma_hstore<kDnPass>(P, nc, rs, tag, hr, t0, t0 + kHalf, &s_bad);
    seg_next(S, 1, R, nst, kDnPass, nc);
    lds_barrier();
  }
  for (int q = 0; q < npos; q += 2) {
    dn_mfma_one<WS>(P, S, tag, R, nst, q, npos, rs, cc, nc, A0, A1, t0, t1, acc, &s_bad);
    if (q + 1 >= npos) break;
    dn_mfma_one<WS>(P, S, tag, R, nst, q + 1, npos, rs, cc, nc, A1, A0, t1, t0, acc, &s_bad);
  }
  return s_bad == 0;  // after the last step's barrier: the same in every wave
}
__device__ __forceinline__ bool down_mfma(const Params& P, const Smem& S, uint32_t tag, int wg, int G) {
  if (P.F % 256 == 0)  // uniform
    return down_mfma_ws<true>(P, S, tag, wg, G);
  return down_mfma_ws<false>(P, S, tag, wg, G);
}

// ---------------------------------------------------------- combine ---------
// out[t][c] = sum over j < k of the tagged gated rows y[t*k + j][c], in slot
// order.  Unit = (token, 64 columns), one wave.
// In a stack (P.stack_layers > 0) the sum goes onto the residual stream:
// r_{l+1} = (layer 0 ? x0 : rin) + sum, written to rout with agent-scope
// (write-through) stores, which the next layer's workgroups read after the
// arrival wait without a write-back of the L2.  Each element of the stream is
// read and written by the same wave in every layer.  Returns false if a wait
// was abandoned (the wave's remaining units are then not written).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite f
}
// The k gated rows of unit u's token at the unit's columns (16-byte loads of
// two tagged words per lane), summed in slot order.  The loads of all k slots,
// of up to two units (U units), are issued before any is used (groups of 8
// slots), so a wave waits for one round trip per group instead of one per
// slot.  ok[i]: every word of unit i carried the call's tag.
constexpr int kCombCols = 2 * kWave;  // two columns (one 16-byte load of tagged words) per lane
template <int U>
__device__ __forceinline__ void combine_sum(const Params& P, uint32_t tag, const int (&u)[U], int nd, float (&a0)[U],
                                            float (&a1)[U], bool (&ok)[U]) {
  const int lane = threadIdx.x & (kWave - 1);
  __amdgpu_buffer_rsrc_t rs[U];
  uint32_t cc[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int t = u[i] / nd, c = (u[i] % nd) * kCombCols + 2 * lane;  // d is even: c < d means c + 1 < d
    rs[i] = make_rsrc(P.yq + (size_t)t * P.k * P.d, (uint32_t)(P.k * P.d) * 8u);
    cc[i] = (uint32_t)min(c, P.d - 2);
    a0[i] = a1[i] = 0.f;
    ok[i] = true;
  }
  for (int j0 = 0; j0 < P.k; j0 += 8) {
    u32x4_t q[U][8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j0 + j < P.k)  // uniform
#pragma unroll
        for (int i = 0; i < U; ++i) q[i][j] = ld_coherent16(rs[i], ((uint32_t)(j0 + j) * P.d + cc[i]) * 8u);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j0 + j < P.k)
#pragma unroll
        for (int i = 0; i < U; ++i) {
          ok[i] &= (q[i][j].y == tag) && (q[i][j].w == tag);
          a0[i] += u2f(q[i][j].x);
          a1[i] += u2f(q[i][j].z);
        }
  }
}

// Writes unit u's sums (see combine_step).
__device__ __forceinline__ void combine_store(const Params& P, int u, int nd, int layer, float a0, float a1) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = u / nd, c = (u % nd) * kCombCols + 2 * lane;
  if (c >= P.d) return;
  float2* o = reinterpret_cast<float2*>(P.out + (size_t)t * P.d + c);
  if (P.stack_layers > 0) {  // uniform
    if (layer == 0) {
      const uint32_t xv = *reinterpret_cast<const uint32_t*>(P.x0 + (size_t)t * P.d + c);
      a0 = bf16lo(xv) + a0;
      a1 = bf16hi(xv) + a1;
    } else {
      const float2 r = *reinterpret_cast<const float2*>(P.rin + (size_t)t * P.d + c);
      a0 = r.x + a0;
      a1 = r.y + a1;
    }
    o = reinterpret_cast<float2*>(P.rout + (size_t)t * P.d + c);
    const uint64_t bits =
        (uint64_t)__builtin_bit_cast(uint32_t, a0) | ((uint64_t)__builtin_bit_cast(uint32_t, a1) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(o), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *o = make_float2(a0, a1);
  }
}

// Unit u until its words are current (polling with the watchdog), then stored.
__device__ __forceinline__ bool combine_wait(const Params& P, uint32_t tag, int u, int nd, int layer) {
  const uint64_t t0 = wall_clock64();
  int round = 0;
  for (;;) {
    const int uu[1] = {u};
    float a0[1], a1[1];
    bool ok[1];
    combine_sum<1>(P, tag, uu, nd, a0, a1, ok);
    if (__all(ok[0])) {
      combine_store(P, u, nd, layer, a0[0], a1[0]);
      return true;
    }
    if (!keep_waiting(P, tag, t0, kSiteY, u, round, 3)) return false;
  }
}

__device__ __forceinline__ bool combine_step(const Params& P, uint32_t tag, int gw, int NW, int layer) {
  const int nd = (P.d + kCombCols - 1) / kCombCols;
  const int nunits = P.T * nd;
  // units gw, gw + NW, ... taken two at a time: one first attempt for both,
  // then whichever is not complete waits on its own
  for (int u = gw; u < nunits; u += 2 * NW) {
    if (u + NW < nunits) {  // uniform
      const int uu[2] = {u, u + NW};
      float a0[2], a1[2];
      bool ok[2];
      combine_sum<2>(P, tag, uu, nd, a0, a1, ok);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (__all(ok[i]))
          combine_store(P, uu[i], nd, layer, a0[i], a1[i]);
        else if (!combine_wait(P, tag, uu[i], nd, layer))
          return false;
      }
    } else if (!combine_wait(P, tag, u, nd, layer)) {
      return false;
    }
  }
  return true;
}

// A wave whose waits were abandoned (a watchdog fired: MOE_ETIMEOUT) writes
// NaN into every out element of the combine units it owns (the units of
// combine_step), so that out never keeps an earlier call's plausible values.
// Units whose combine completed hold this call's correct sums: every tagged
// word a combine accepts was computed from complete inputs, because a step
// whose wait was abandoned stores no tagged results.
__device__ __forceinline__ void poison_out(const Params& P, float* dst, int gw, int NW) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nd = (P.d + kCombCols - 1) / kCombCols;
  const float nan = __builtin_nanf("");
  for (int u = gw; u < P.T * nd; u += NW) {
    const int t = u / nd, c = (u % nd) * kCombCols + 2 * lane;
    if (c < P.d) *reinterpret_cast<float2*>(dst + (size_t)t * P.d + c) = make_float2(nan, nan);
  }
}

// ---------------------------------------------------------- kernels ---------

// Expert-step variants of the whole-layer kernel (the host picks one, see
// plan_launch): kVAll, x of every token in LDS (two W_down chunks per lane);
// kVAllH, the same with the down step's h staged per workgroup where it pays
// (stage_h: experts of more than two tokens, or few units per workgroup; one
// W_down chunk per lane); kVPairs, x of each workgroup's own pairs in LDS and
// h staged; kVMfma, the MFMA expert steps.
constexpr int kVAll = 0, kVAllH = 1, kVPairs = 2, kVMfma = 3;

// The whole layer in one launch.  V: variant; MM: W_down chunks per lane.
template <int V, int MM>
__global__ void __launch_bounds__(kWG) k_layer(Params P) {
  constexpr bool SMALL = V != kVMfma, XP = V == kVPairs, HS = V == kVAllH || V == kVPairs;
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_ok;
  const Smem S = carve(smem, P, SMALL);
  const int wg = blockIdx.x, G = gridDim.x;
  const int gw = wg * kWaves + uni(threadIdx.x / kWave), NW = G * kWaves;
  const uint32_t tag = start_call(P, wg, true);
  stamp(P, wg, 0);
  if (threadIdx.x == 0) s_ok = 1;
  if (P.T > kRouterMfmaT)
    router_mfma(P, tag, wg, G, S.rt);
  else
    router_step<false>(P, S, tag, wg, G, [] {});
  stamp(P, wg, 1);
  bool ok = topk_publish(P, tag, gw, NW);
  stamp(P, wg, 7);
  // x into LDS while the top-k results are on their way (owner waves first)
  if (SMALL && !XP) stage_x(P, S.xs, P.T, [](int r) { return r; });
  __syncthreads();
  ok = load_topk(P, S, tag, wg % kTopkRep) && ok;
  __syncthreads();
  if (!ok) s_ok = 0;
  __syncthreads();
  stamp(P, wg, 2);
  if (s_ok) {
    build_perm(P, S, wg == 0);
    set_ranges(P, S, wg, G);
    if (XP) stage_pairs(P, S);
    stamp(P, wg, 3);
    bool dn = true;
    // Before the down step's cached first reads of h, the L2 of every XCD
    // drops its lines of earlier calls: one wave of workgroups 0-7 (one per
    // XCD, as workgroups are dealt to the XCDs in turn; were it otherwise, a
    // stale line only sends its readers to the coherent path).  Its own
    // gate/up loads wait for it, the other waves' do not.
    if (wg < 8 && threadIdx.x >= kWG - kWave) invalidate_l2();
    if (SMALL) {
      gate_up_waves<XP>(P, S, tag, wg, G);
      stamp(P, wg, 4);
      stamp_gu_wave(P, wg);
      dn = down_dispatch<MM, HS, !XP>(P, S, tag, wg, G, (size_t)P.xrows * P.d * 2);
    } else {
      gate_up_mfma(P, S, tag, wg, G);
      stamp(P, wg, 4);
      dn = down_mfma(P, S, tag, wg, G);
    }
    stamp(P, wg, 5);
    if (dn) dn = combine_step(P, tag, gw, NW, P.layer0);
    stamp(P, wg, 6);
    if (!dn) poison_out(P, P.stack_layers > 0 ? P.rout : P.out, gw, NW);
  } else {
    poison_out(P, P.stack_layers > 0 ? P.rout : P.out, gw, NW);
  }
  __syncthreads();
  if (wg == 0) end_call(P, tag, G);
}

// ------------------------------------------------- normalised layer input --
// Input of a layer of a stack: x_l = bf16(r_l / sqrt(mean(r_l^2) + eps)),
// unit gain, eps = 1e-6, round to nearest even ([P3-PK] lists the
// normalisation among the operators between layers).  r_l is fp32 [T][d] at
// rf, or for layer 0 the stack's bf16 input rb.  Rows t0..t1-1 in groups of
// kNormRows, by the whole workgroup: thread i holds the row's 8-element pieces
// i and i + kWG (d <= 8192) of every row of the group in registers (one round
// of loads per group), sums their squares in order, each wave adds its lanes
// in a fixed butterfly and the 8 wave sums are added in wave order, so every
// workgroup that normalises a row (and k_norm) gets the same bits.  A scaled
// piece goes to the piece-transposed LDS rows of stage_x (xs, row t - t0)
// and/or to row t of xg (bf16, row-major).  All threads.  (Groups of 2 rows:
// 4 rows in flight pushed the resident stack kernel's registers into scratch.)
constexpr float kStackEps = 1e-6f;
constexpr int kNormRows = 2;
__device__ void norm_rows(const Params& P, const float* rf, const uint16_t* rb, int t0, int t1, u32x4_t* xs,
                          uint16_t* xg) {
  __shared__ float s_ss[kNormRows][kWaves];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int NCH = P.d / 32, npc = P.d / 8;
  const int i0 = threadIdx.x, i1 = threadIdx.x + kWG;
  const bool h0 = i0 < npc, h1 = i1 < npc;  // pieces this thread holds
  for (int g0 = t0; g0 < t1; g0 += kNormRows) {
    const int ng = min(kNormRows, t1 - g0);
    float v[kNormRows][2][8];
    // loads: every row of the group, both pieces (absent ones read piece 0
    // and are not used)
#pragma unroll
    for (int r = 0; r < kNormRows; ++r) {
      const int t = g0 + min(r, ng - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = (h == 0 ? h0 : h1) ? (h == 0 ? i0 : i1) : 0;
        if (rb != nullptr) {  // uniform
          const u32x4_t q = *reinterpret_cast<const u32x4_t*>(rb + (size_t)t * P.d + 8 * i);
          v[r][h][0] = bf16lo(q.x); v[r][h][1] = bf16hi(q.x); v[r][h][2] = bf16lo(q.y); v[r][h][3] = bf16hi(q.y);
          v[r][h][4] = bf16lo(q.z); v[r][h][5] = bf16hi(q.z); v[r][h][6] = bf16lo(q.w); v[r][h][7] = bf16hi(q.w);
        } else {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(rf + (size_t)t * P.d + 8 * i);
          const u32x4_t b = *reinterpret_cast<const u32x4_t*>(rf + (size_t)t * P.d + 8 * i + 4);
          v[r][h][0] = u2f(a.x); v[r][h][1] = u2f(a.y); v[r][h][2] = u2f(a.z); v[r][h][3] = u2f(a.w);
          v[r][h][4] = u2f(b.x); v[r][h][5] = u2f(b.y); v[r][h][6] = u2f(b.z); v[r][h][7] = u2f(b.w);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kNormRows; ++r) {
      float ss = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (h == 0 ? h0 : h1)
#pragma unroll
          for (int j = 0; j < 8; ++j) ss = fmaf(v[r][h][j], v[r][h][j], ss);
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
      if (lane == 0) s_ss[r][wave] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kNormRows; ++r) {
      if (r < ng) {  // uniform
        const int t = g0 + r;
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += s_ss[r][w];
        const float inv = 1.f / sqrtf(tot / (float)P.d + kStackEps);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 0 ? h0 : h1) {
            const int i = h == 0 ? i0 : i1;
            u32x4_t q;
            q.x = bf16_rne(v[r][h][0] * inv) | (bf16_rne(v[r][h][1] * inv) << 16);
            q.y = bf16_rne(v[r][h][2] * inv) | (bf16_rne(v[r][h][3] * inv) << 16);
            q.z = bf16_rne(v[r][h][4] * inv) | (bf16_rne(v[r][h][5] * inv) << 16);
            q.w = bf16_rne(v[r][h][6] * inv) | (bf16_rne(v[r][h][7] * inv) << 16);
            if (xs != nullptr) xs[(size_t)(t - t0) * 4 * NCH + (i % 4) * NCH + i / 4] = q;
            if (xg != nullptr) *reinterpret_cast<u32x4_t*>(xg + (size_t)t * P.d + 8 * i) = q;
          }
        }
      }
    }
    __syncthreads();  // s_ss is reused by the next group
  }
}

// One launch per layer: the layer's input, one row per workgroup.
__global__ void __launch_bounds__(kWG) k_norm(Params P) {
  const bool first = P.layer0 == 0;
  norm_rows(P, first ? nullptr : P.out, first ? P.x0 : nullptr, blockIdx.x, blockIdx.x + 1, nullptr, P.xb);
}

// ------------------------------------------------- a stack in one launch ---
// Layer after layer of a stack inside one resident launch ([P3-PK]: the
// pipeline stays on the GPU, no return to the host between operators;
// [P5-TRT]: MoE gate then expert compute, per layer).  Layer l runs under tag
// t0 + l.  Between layers every workgroup publishes its part of the stream r
// (the combine's stores into out or rbuf, alternating by layer, agent-scope
// atomics that write through the L2; each
// wave waits for them to complete, so no L2 write-back is needed: one per wave
// cost ~45 us per layer), then its arrival word (hdr[kStarted + wg]) takes
// the next layer's tag.  The next layer's router needs the input of every
// token, so each workgroup waits until every arrival word has reached that
// tag, acquires (dropping its CU's and XCD's stale lines) and normalises r
// into its LDS itself (every workgroup gets the same bits, see norm_rows).
// The router's first weight loads are already in flight during the wait.
// Measured on MI355X (8 verify-block layers): one launch ~268 us per layer,
// one launch per operator ~250 us: back-to-back launches on one stream leave
// no measurable gap between kernels, and this kernel's layer loop costs
// registers (its hot loops reload some spilled values from scratch).

// Tags of this launch lie in [t0, t0 + nl): a raised abort word in that range
// stops the stack.
__device__ __forceinline__ bool stack_aborted(const Params& P, uint32_t t0) {
  return ld_relaxed(&P.hdr[kAbort]) - t0 < (uint32_t)P.nlayers;
}

// Wave 0: every workgroup's arrival word has reached `tag` (a signed
// difference, so that the words of earlier launches, including those from
// before the tags restarted at 1, count as behind it).  False if the wait was
// abandoned.
__device__ __forceinline__ bool wait_arrivals(const Params& P, uint32_t t0, uint32_t tag, int G) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t ts = wall_clock64();
  int round = 0;
  for (;;) {
    bool ok = true;
    for (int w = lane; w < G; w += kWave) ok &= (int32_t)(ld_relaxed(&P.hdr[kStarted + w]) - tag) >= 0;
    if (__all(ok)) return true;
    if ((round & 7) == 7 && stack_aborted(P, t0)) return false;
    if (wall_clock64() - ts > P.spin_ticks) {
      if (lane == 0) raise_timeout(P, tag, kSiteLayer, 0);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
    ++round;
    __asm__ __volatile__("" ::: "memory");
  }
}

template <int V, int MM>
__global__ void __launch_bounds__(kWG) k_stack(Params P0) {
  static_assert(V == kVAll || V == kVAllH, "stacks keep x of every token in LDS");
  constexpr bool HS = V == kVAllH;
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_ok, s_go;
  const Smem S = carve(smem, P0, true);
  const int wg = blockIdx.x, G = gridDim.x;
  const int gw = wg * kWaves + uni(threadIdx.x / kWave), NW = G * kWaves;
  const uint32_t t0 = start_call(P0, wg, true, P0.nlayers);
  const uint32_t tlast = t0 + (uint32_t)P0.nlayers - 1u;
  Params P = P0;
  int l = 0;
  uint32_t tag = t0;
  int sl = P0.layer0;
  bool failed = false;
  // The layer loop is entered at its top, and (never: the host passes
  // nlayers >= 1) at its second half: a cycle with two entries is not a
  // natural loop, so the optimizer hoists none of the body's lane-invariant
  // values out of it, which would hold them in registers across the whole
  // layer (measured: ~190 VGPR spills with the plain loop, none without).
  if (P0.nlayers < 1) goto second_half;
  for (;;) {
    tag = t0 + (uint32_t)l;
    sl = P0.layer0 + l;
    P.wr = P0.wr + (size_t)l * P0.wr_stride;
    P.packed = P0.packed + (size_t)l * P0.pk_stride;
    P.scales = P0.scales + (size_t)l * P0.sc_stride;
    // The stream alternates between two buffers: layer sl writes r_{sl+1} to
    // out if L - 1 - sl is even, else to rbuf (so the last layer's lands in
    // out), and reads r_sl where layer sl - 1 wrote it.  A buffer is written
    // again only two layers after it was read, i.e. after every workgroup's
    // arrival at the layer in between, so a workgroup still normalising r_sl
    // never sees it overwritten.  (With one buffer, a workgroup whose results
    // nothing waited for could still be reading r_sl while others already
    // wrote r_{sl+1} over it.)
    P.rout = ((P0.stack_layers - 1 - sl) & 1) ? P0.rbuf : P0.out;
    P.rin = ((P0.stack_layers - sl) & 1) ? P0.rbuf : P0.out;
    if (threadIdx.x == 0) s_ok = s_go = 1;
    __syncthreads();
    router_step<true>(P, S, tag, wg, G, [&] {
      if (l > 0) {
        if (threadIdx.x < kWave) {
          const bool ok = wait_arrivals(P, t0, tag, G);
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          if (!ok && threadIdx.x == 0) s_go = 0;
        }
        __syncthreads();
      }
      // workgroup 0 also leaves the last layer's input in xb, for inspection
      if (s_go)
        norm_rows(P, sl == 0 ? nullptr : P.rin, sl == 0 ? P.x0 : nullptr, 0, P.T, S.xs,
                  (wg == 0 && l == P0.nlayers - 1) ? P0.xb : nullptr);
      __syncthreads();
    });
    if (!s_go) {  // uniform
      failed = true;
      break;
    }
  second_half:
    {
      bool ok = topk_publish(P, tag, gw, NW);
      __syncthreads();
      ok = load_topk(P, S, tag, wg % kTopkRep) && ok;
      __syncthreads();
      if (!ok) s_ok = 0;
      __syncthreads();
      if (!s_ok) {  // uniform
        failed = true;
        break;
      }
      build_perm(P, S, wg == 0);
      set_ranges(P, S, wg, G);
      if (wg < 8 && threadIdx.x >= kWG - kWave) invalidate_l2();
      gate_up_waves<false>(P, S, tag, wg, G);
      bool dn = down_dispatch<MM, HS, true>(P, S, tag, wg, G, (size_t)P.xrows * P.d * 2);
      if (dn) dn = combine_step(P, tag, gw, NW, sl);
      if (!dn) s_ok = 0;
      // this wave's write-through stores of r have completed before the arrival
      __builtin_amdgcn_s_waitcnt(0);
      if (threadIdx.x == 0 && stack_aborted(P0, t0)) s_ok = 0;
      __syncthreads();
      if (!s_ok) {  // uniform
        failed = true;
        break;
      }
    }
    if (++l >= P0.nlayers) break;
    if (threadIdx.x == 0) st_relaxed(&P0.hdr[kStarted + wg], tag + 1u);
  }
  // a stack stopped by an abandoned wait leaves NaN in the out elements of
  // the workgroup's combine units (see poison_out)
  if (failed) poison_out(P0, P0.out, gw, NW);
  // a workgroup that stopped early still closes its arrival word, so that
  // the end of the launch does not wait for it
  __syncthreads();
  if (threadIdx.x == 0) st_relaxed(&P0.hdr[kStarted + wg], tlast);
  __syncthreads();
  if (wg == 0) end_call(P0, tlast, G);
}

// One launch per step (the per-operator model), same arithmetic.
__global__ void __launch_bounds__(kWG) k_st_router(Params P) {
  extern __shared__ __align__(16) char smem[];  // kRouterTileBytes for more than kRouterMfmaT tokens
  const uint32_t tag = start_call(P, blockIdx.x, false);
  if (P.T > kRouterMfmaT)
    router_mfma(P, tag, blockIdx.x, gridDim.x, reinterpret_cast<float*>(smem));
  else
    router_step<false>(P, Smem{}, tag, blockIdx.x, gridDim.x, [] {});
}
__global__ void __launch_bounds__(kWG) k_st_topk(Params P) {
  const uint32_t tag = start_call(P, blockIdx.x, false);
  topk_publish(P, tag, blockIdx.x * kWaves + uni(threadIdx.x / kWave), gridDim.x * kWaves);
}
__global__ void __launch_bounds__(kWG) k_st_perm(Params P) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_ok;
  const Smem S = carve(smem, P, false);
  const uint32_t tag = start_call(P, blockIdx.x, false);
  if (threadIdx.x == 0) s_ok = 1;
  __syncthreads();
  if (!load_topk(P, S, tag, blockIdx.x % kTopkRep)) s_ok = 0;
  __syncthreads();
  if (s_ok) build_perm(P, S, true);
}
template <bool SMALL>
__global__ void __launch_bounds__(kWG) k_st_gate_up(Params P) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_ok;
  const Smem S = carve(smem, P, SMALL);
  const uint32_t tag = start_call(P, blockIdx.x, false);
  if (threadIdx.x == 0) s_ok = 1;
  __syncthreads();
  if (!load_topk(P, S, tag, blockIdx.x % kTopkRep)) s_ok = 0;
  __syncthreads();
  if (!s_ok) return;
  build_perm(P, S, false);
  set_ranges(P, S, blockIdx.x, gridDim.x);
  if (SMALL) {
    if (P.xmode == 0) {
      stage_x(P, S.xs, P.T, [](int r) { return r; });
      __syncthreads();
      gate_up_waves<false>(P, S, tag, blockIdx.x, gridDim.x);
    } else {
      stage_pairs(P, S);
      gate_up_waves<true>(P, S, tag, blockIdx.x, gridDim.x);
    }
  } else {
    gate_up_mfma(P, S, tag, blockIdx.x, gridDim.x);
  }
}
// MM: W_down chunks per lane of the small-batch path; 0 = the MFMA path.
template <int MM>
__global__ void __launch_bounds__(kWG) k_st_down(Params P) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_ok;
  const Smem S = carve(smem, P, false);
  const uint32_t tag = start_call(P, blockIdx.x, false);
  if (threadIdx.x == 0) s_ok = 1;
  __syncthreads();
  if (!load_topk(P, S, tag, blockIdx.x % kTopkRep)) s_ok = 0;
  __syncthreads();
  if (!s_ok) return;
  build_perm(P, S, false);
  set_ranges(P, S, blockIdx.x, gridDim.x);
  if (threadIdx.x < kWave) invalidate_l2();  // before the cached first reads of h
  if (MM == 0) {
    down_mfma(P, S, tag, blockIdx.x, gridDim.x);
  } else {
    // the x area of this layout: the MFMA tiles or the masks, whichever is larger
    const LdsPlan L = lds_plan(P.T, P.d, P.E, P.k, 0);
    if (P.xmode == 0)
      down_dispatch<MM == 0 ? 1 : MM, true, true>(P, S, tag, blockIdx.x, gridDim.x, L.tki - L.xs);
    else
      down_dispatch<MM == 0 ? 1 : MM, true, false>(P, S, tag, blockIdx.x, gridDim.x, L.tki - L.xs);
  }
}
__global__ void __launch_bounds__(kWG) k_st_combine(Params P) {
  const uint32_t tag = start_call(P, blockIdx.x, false);
  const int gw = blockIdx.x * kWaves + uni(threadIdx.x / kWave), NW = gridDim.x * kWaves;
  if (!combine_step(P, tag, gw, NW, P.layer0)) poison_out(P, P.stack_layers > 0 ? P.rout : P.out, gw, NW);
}
__global__ void k_st_bump(Params P) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const uint32_t e = ld_relaxed(&P.hdr[kEpoch]);
    st_relaxed(&P.hdr[kEpoch], next_epoch(e + 1u));
  }
}
__global__ void k_zero(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ------------------------------------------------------------ host side -----

constexpr size_t kAlign = 256;
static inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

static int check_dims(const moe_mxfp4_dims* dm, int32_t topk) {
  if (!dm) return MOE_EINVAL;
  if (dm->T < 0 || dm->E < 1 || topk < 1 || topk > dm->E) return MOE_EINVAL;
  if (dm->E > kMaxE || topk > kMaxK) return MOE_ESHAPE;
  if (dm->d < 32 || dm->ffn < 32 || dm->d % 32 || dm->ffn % 32) return MOE_ESHAPE;
  if (dm->d > kMaxD || dm->ffn > kMaxF) return MOE_ESHAPE;
  const int64_t W = ((int64_t)dm->T + 63) / 64;
  if ((int64_t)dm->E * W > kMaxMaskWords) return MOE_ESHAPE;
  return MOE_OK;
}

struct Layout {
  size_t hdr, lgp, tk, hq, yq, logits, topk_idx, topk_w, offsets, sorted_slot, pos, active, n_active, trace, xb,
      rb, total;
};

static Layout make_layout(const moe_mxfp4_dims* dm, int32_t k) {
  Layout L;
  const size_t T = (size_t)dm->T, E = (size_t)dm->E, TK = T * (size_t)k;
  size_t o = 0;
  L.hdr = o; o = align_up(o + kHdrBytes);
  // two arrays of partial logits where the MFMA router splits K (router_halves)
  L.lgp = o; o = align_up(o + (T > (size_t)kRouterMfmaT ? 2 : 1) * T * ((E + 1) & ~(size_t)1) * 8);
  L.tk = o; o = align_up(o + (size_t)kTopkRep * TK * 16);
  L.hq = o; o = align_up(o + TK * (size_t)dm->ffn * 8);
  L.yq = o; o = align_up(o + TK * (size_t)dm->d * 8);
  L.logits = o; o = align_up(o + T * E * 4);
  L.topk_idx = o; o = align_up(o + TK * 4);
  L.topk_w = o; o = align_up(o + TK * 4);
  L.offsets = o; o = align_up(o + (E + 1) * 4);
  L.sorted_slot = o; o = align_up(o + TK * 4);
  L.pos = o; o = align_up(o + TK * 4);
  L.active = o; o = align_up(o + E * 4);
  L.n_active = o; o = align_up(o + 4);
  L.trace = o; o = align_up(o + (size_t)kMaxGrid * kTraceSlots * 8);
  L.xb = o; o = align_up(o + T * (size_t)dm->d * 2);
  L.rb = o; o = align_up(o + T * (size_t)dm->d * 4);
  L.total = o;
  return L;
}

// x of all tokens fits in LDS next to the permutation tables.
// Rows of x the small-batch path's LDS can hold next to its tables.
static int x_rows_fit(const moe_mxfp4_dims* dm, int32_t k) {
  const size_t tables = lds_plan(dm->T, dm->d, dm->E, k, 1).total - al16((size_t)dm->d * 2);
  if (tables >= (size_t)kLdsMax) return 0;
  return (int)(((size_t)kLdsMax - tables) / ((size_t)dm->d * 2));
}


struct DeviceInfo {
  int cus = 0;
  uint64_t ticks_per_us = 100;
  bool ok = false;
};

static std::mutex g_mu;
static DeviceInfo g_info[64];

static const void* layer_kernel(int v, int mm) {
  switch (v) {
    case kVAll: return (const void*)k_layer<kVAll, 2>;    // mm 2 only: mm 1 takes kVAllH (plan_launch)
    case kVAllH: return (const void*)k_layer<kVAllH, 1>;  // the static down path (mm 2) stages nothing
    case kVPairs: return mm == 1 ? (const void*)k_layer<kVPairs, 1> : (const void*)k_layer<kVPairs, 2>;
    default: return mm == 1 ? (const void*)k_layer<kVMfma, 1> : (const void*)k_layer<kVMfma, 2>;
  }
}

// The one-launch stack: small-batch path with x of every token in LDS.
static const void* stack_kernel(int v, int mm) {
  if (v == kVAllH) return (const void*)k_stack<kVAllH, 1>;
  if (v == kVAll) return (const void*)k_stack<kVAll, 2>;
  (void)mm;
  return nullptr;
}

static int device_info(DeviceInfo* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_EDEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceInfo& di = g_info[dev];
  if (!di.ok) {
    int cus = 0, khz = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_EDEVICE;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return MOE_EDEVICE;
    const void* ks[] = {layer_kernel(kVAll, 2), layer_kernel(kVAllH, 1),
                        layer_kernel(kVPairs, 1), layer_kernel(kVPairs, 2), layer_kernel(kVMfma, 1),
                        layer_kernel(kVMfma, 2), stack_kernel(kVAll, 2), stack_kernel(kVAllH, 1),
                        (const void*)k_st_perm, (const void*)k_st_gate_up<true>, (const void*)k_st_gate_up<false>,
                        (const void*)k_st_down<0>, (const void*)k_st_down<1>, (const void*)k_st_down<2>};
    for (const void* f : ks) {
      if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax) != hipSuccess) {
        (void)hipGetLastError();  // do not leave a sticky error for the caller's next HIP call
        return MOE_EDEVICE;
      }
    }
    di.cus = cus;
    di.ticks_per_us = khz >= 1000 ? (uint64_t)khz / 1000u : 100u;
    di.ok = true;
  }
  *out = di;
  return MOE_OK;
}

static int check_io_ptrs(const void* x, const float* wr, const uint8_t* packed, const uint8_t* scales,
                         const float* out) {
  if (!x || !wr || !packed || !scales || !out) return MOE_EINVAL;
  auto al = [](const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; };
  if (!al(x, 16) || !al(wr, 16) || !al(packed, 16) || !al(out, 16)) return MOE_EALIGN;
  return MOE_OK;
}

static int check_ptrs(const void* x, const float* wr, const uint8_t* packed, const uint8_t* scales, const float* out,
                      const void* ws) {
  const int st = check_io_ptrs(x, wr, packed, scales, out);
  if (st != MOE_OK) return st;
  if (!ws) return MOE_EINVAL;
  if ((uintptr_t)ws % kAlign) return MOE_EALIGN;
  return MOE_OK;
}

static Params make_params(const moe_mxfp4_dims* dm, int32_t k, const void* x, const float* wr, const uint8_t* packed,
                          const uint8_t* scales, float* out, void* ws, const DeviceInfo& di, uint32_t spin_us) {
  const Layout L = make_layout(dm, k);
  char* b = static_cast<char*>(ws);
  Params P;
  P.T = dm->T;
  P.d = dm->d;
  P.F = dm->ffn;
  P.E = dm->E;
  P.k = k;
  P.x = static_cast<const uint16_t*>(x);
  P.wr = wr;
  P.packed = packed;
  P.scales = scales;
  P.out = out;
  P.hdr = reinterpret_cast<uint32_t*>(b + L.hdr);
  P.lgp = reinterpret_cast<uint64_t*>(b + L.lgp);
  P.tk = reinterpret_cast<uint64_t*>(b + L.tk);
  P.hq = reinterpret_cast<uint64_t*>(b + L.hq);
  P.yq = reinterpret_cast<uint64_t*>(b + L.yq);
  P.logits = reinterpret_cast<float*>(b + L.logits);
  P.topk_idx = reinterpret_cast<int32_t*>(b + L.topk_idx);
  P.topk_w = reinterpret_cast<float*>(b + L.topk_w);
  P.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  P.sorted_slot = reinterpret_cast<int32_t*>(b + L.sorted_slot);
  P.pos = reinterpret_cast<int32_t*>(b + L.pos);
  P.active = reinterpret_cast<int32_t*>(b + L.active);
  P.n_active = reinterpret_cast<int32_t*>(b + L.n_active);
  P.trace = nullptr;
  const uint64_t us = spin_us ? spin_us : 2000000u;
  P.spin_ticks = us * di.ticks_per_us;
  P.withhold = 0;
  P.withhold_h = 0;
  P.mfma = 0;
  P.xmode = 0;
  P.xrows = 0;
  P.narrow = (size_t)dm->T * k * (size_t)(dm->d > dm->ffn ? dm->d : dm->ffn) * 8 < ((size_t)1 << 32) ? 1 : 0;
  P.stack_layers = 0;
  P.layer0 = 0;
  P.nlayers = 1;
  P.xb = reinterpret_cast<uint16_t*>(b + L.xb);
  P.x0 = static_cast<const uint16_t*>(x);
  P.rin = out;
  P.rout = out;
  P.rbuf = reinterpret_cast<float*>(b + L.rb);
  P.wr_stride = P.pk_stride = P.sc_stride = 0;
  return P;
}

static int chunks_per_lane_down(const moe_mxfp4_dims* dm) { return (dm->ffn / 32 + kWave - 1) / kWave; }

static int grid_for(const DeviceInfo& di, const void* kern, size_t lds, int requested) {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kWG, lds) != hipSuccess || occ < 1) {
    (void)hipGetLastError();
    occ = 1;
  }
  int maxg = di.cus * occ;
  if (maxg > kMaxGrid) maxg = kMaxGrid;
  int g = di.cus < maxg ? di.cus : maxg;  // one workgroup per CU
  if (requested > 0) g = requested < maxg ? requested : maxg;
  return g < 1 ? 1 : g;
}

struct Launch {
  bool small;
  int mm;
  size_t lds;
  int xmode, xrows;
  int v;  // kernel variant
};

// Expert-step path: x of every token in LDS (small-batch VALU path, xmode 0);
// else, up to kPairMaxT tokens, the x rows of each workgroup's own pairs
// (xmode 1: a few experts per workgroup, about T*k/n_active tokens each);
// else the MFMA path.
constexpr int kPairMaxT = 48;
static int plan_launch(const moe_mxfp4_dims* dm, int32_t k, Launch* L) {
  const int fit = x_rows_fit(dm, k);
  L->small = true;
  L->xmode = 0;
  L->xrows = dm->T;
  if (fit < dm->T) {
    if (dm->T <= kPairMaxT && fit >= 4) {
      L->xmode = 1;
      L->xrows = fit;
    } else {
      L->small = false;
      L->xrows = 0;
    }
  }
  L->mm = chunks_per_lane_down(dm);
  if (L->mm < 1 || L->mm > 2) return MOE_ESHAPE;
  // x of every token in LDS: with one W_down chunk per lane the down step may
  // stage h per workgroup (kVAllH), which pays where an expert has more than
  // two tokens (the waves would reload h per pass: measured 320 instead of
  // 240 us for a verify block with one 3-token expert) or a workgroup has few
  // down units; otherwise it costs ~1% (verify, at most 2 tokens per expert:
  // 249 instead of 247 us)
  L->v = !L->small ? kVMfma : L->xmode == 1 ? kVPairs : L->mm == 1 ? kVAllH : kVAll;
  const LdsPlan pl = lds_plan(dm->T, dm->d, dm->E, k, L->xrows);
  if (pl.total > (size_t)kLdsMax) return MOE_ESHAPE;
  L->lds = pl.total;
  return MOE_OK;
}

static void apply_launch(Params& P, const Launch& L) {
  P.mfma = L.small ? 0 : 1;
  P.xmode = L.xmode;
  P.xrows = L.xrows;
}

// The layer's waits need every workgroup resident at once.  The grid is at
// most one workgroup per CU and a workgroup's registers and LDS fill a CU, so
// on an idle device a plain launch places them all; a cooperative launch
// guarantees it but costs ~17 us more per call on MI355X (measured: 19 us vs
// 2.3 us back to back for an empty kernel), so it is an option.  If other work
// holds CUs, a plain launch's waits time out (MOE_ETIMEOUT) instead of hanging.
static int launch_layer(Params P, const Launch& L, int grid, hipStream_t s, bool cooperative) {
  void* args[] = {&P};
  hipError_t e;
  if (cooperative)
    e = hipLaunchCooperativeKernel(layer_kernel(L.v, L.mm), dim3(grid), dim3(kWG), args, (unsigned)L.lds, s);
  else
    e = hipLaunchKernel(layer_kernel(L.v, L.mm), dim3(grid), dim3(kWG), args, (unsigned)L.lds, s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ELAUNCH;
  }
  return MOE_OK;
}

static int launch_staged(const Params& P, const Launch& L, int grid, hipStream_t s, bool experts) {
  const unsigned lds_tables = (unsigned)lds_plan(P.T, P.d, P.E, P.k, 0).total;
  hipLaunchKernelGGL(k_st_router, dim3(grid), dim3(kWG), P.T > kRouterMfmaT ? kRouterTileBytes : 0, s, P);
  hipLaunchKernelGGL(k_st_topk, dim3(grid), dim3(kWG), 0, s, P);
  if (experts) {
    if (L.small)
      hipLaunchKernelGGL(k_st_gate_up<true>, dim3(grid), dim3(kWG), (unsigned)L.lds, s, P);
    else
      hipLaunchKernelGGL(k_st_gate_up<false>, dim3(grid), dim3(kWG), (unsigned)L.lds, s, P);
    if (!L.small)
      hipLaunchKernelGGL(k_st_down<0>, dim3(grid), dim3(kWG), lds_tables, s, P);
    else if (L.mm == 1)
      hipLaunchKernelGGL(k_st_down<1>, dim3(grid), dim3(kWG), lds_tables, s, P);
    else
      hipLaunchKernelGGL(k_st_down<2>, dim3(grid), dim3(kWG), lds_tables, s, P);
    hipLaunchKernelGGL(k_st_combine, dim3(grid), dim3(kWG), 0, s, P);
  }
  // the permutation copies for inspection come from one workgroup
  hipLaunchKernelGGL(k_st_perm, dim3(1), dim3(kWG), lds_tables, s, P);
  hipLaunchKernelGGL(k_st_bump, dim3(1), dim3(64), 0, s, P);
  if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
  return MOE_OK;
}

// ------------------------------------------------- allocation-free calls ---
// moe_mxfp4_forward_noalloc runs the layer on a workspace that is a
// file-scope device array instead of a caller buffer.  Each device the
// library runs on holds its own copy (kScratchBytes) until the process ends.
// In host code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct ScratchInfo {
  void* ptr = nullptr;
  bool cleared = false;
};
static ScratchInfo g_scratch[64];

// This device's scratch address (set up on first use, with the device
// current); the first call also enqueues a zero fill of it on `s`, ahead of
// the layer kernel that will use it.
static int scratch_for_device(hipStream_t s, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_EDEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  ScratchInfo& si = g_scratch[dev];
  if (si.ptr == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return MOE_EDEVICE;
    }
    si.ptr = ptr;
  }
  if (!si.cleared) {
    hipLaunchKernelGGL(k_zero, dim3(1024), dim3(256), 0, s, static_cast<uint4*>(si.ptr), kScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    si.cleared = true;
  }
  *out = si.ptr;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_mxfp4_expert_packed_bytes(int32_t d, int32_t ffn) {
  if (d <= 0 || ffn <= 0) return 0;
  return (size_t)3 * (size_t)d * (size_t)ffn / 2;
}

size_t moe_mxfp4_expert_scale_bytes(int32_t d, int32_t ffn) {
  if (d <= 0 || ffn <= 0) return 0;
  return (size_t)3 * (size_t)d * (size_t)ffn / 32;
}

size_t moe_mxfp4_workspace_bytes(const moe_mxfp4_dims* dims, int32_t topk) {
  if (check_dims(dims, topk) != MOE_OK) return 0;
  return make_layout(dims, topk).total;
}

int moe_mxfp4_workspace_layout(const moe_mxfp4_dims* dims, int32_t topk, moe_mxfp4_ws_layout* out) {
  int st = check_dims(dims, topk);
  if (st != MOE_OK) return st;
  if (!out) return MOE_EINVAL;
  const Layout L = make_layout(dims, topk);
  out->logits = L.logits;
  out->topk_idx = L.topk_idx;
  out->topk_w = L.topk_w;
  out->offsets = L.offsets;
  out->sorted_slot = L.sorted_slot;
  out->pos = L.pos;
  out->active = L.active;
  out->n_active = L.n_active;
  out->h = L.hq;
  out->y = L.yq;
  out->trace = L.trace;
  out->x_last = L.xb;
  Launch Lp;
  out->h_chunk_major = plan_launch(dims, topk, &Lp) == MOE_OK && Lp.small && Lp.xmode == 0 ? 1 : 0;
  out->total = L.total;
  return MOE_OK;
}

int moe_mxfp4_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return MOE_EINVAL;
  if (workspace_bytes < kHdrBytes) return MOE_EWORKSPACE;
  if ((uintptr_t)workspace % kAlign) return MOE_EALIGN;
  hipLaunchKernelGGL(k_zero, dim3(1024), dim3(256), 0, (hipStream_t)stream, (uint4*)workspace,
                     workspace_bytes / 16);
  if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
  return MOE_OK;
}

int moe_mxfp4_persistent_grid(const moe_mxfp4_dims* dims, int32_t topk) {
  int st = check_dims(dims, topk);
  if (st != MOE_OK) return -st;
  Launch L;
  st = plan_launch(dims, topk, &L);
  if (st != MOE_OK) return -st;
  DeviceInfo di;
  st = device_info(&di);
  if (st != MOE_OK) return -st;
  return grid_for(di, layer_kernel(L.v, L.mm), L.lds, 0);
}

int moe_mxfp4_forward_ex(const moe_mxfp4_dims* dims, const void* x, const float* router_w,
                         const uint8_t* packed_experts, const uint8_t* scales, int32_t topk, float* out,
                         void* workspace, size_t workspace_bytes, const moe_mxfp4_options* opts, void* stream) {
  int st = check_dims(dims, topk);
  if (st != MOE_OK) return st;
  if (opts && (opts->flags & ~(MOE_OPT_WITHHOLD_ARRIVAL | MOE_OPT_TRACE | MOE_OPT_COOPERATIVE | MOE_OPT_WITHHOLD_H)))
    return MOE_EINVAL;
  if (opts && opts->grid < 0) return MOE_EINVAL;
  if (dims->T == 0) return MOE_OK;  // nothing to do; buffers may be empty (null)
  st = check_ptrs(x, router_w, packed_experts, scales, out, workspace);
  if (st != MOE_OK) return st;
  if (workspace_bytes < make_layout(dims, topk).total) return MOE_EWORKSPACE;
  Launch L;
  st = plan_launch(dims, topk, &L);
  if (st != MOE_OK) return st;
  DeviceInfo di;
  st = device_info(&di);
  if (st != MOE_OK) return st;
  Params P = make_params(dims, topk, x, router_w, packed_experts, scales, out, workspace, di,
                         opts ? opts->spin_limit_us : 0u);
  apply_launch(P, L);
  if (opts && (opts->flags & MOE_OPT_WITHHOLD_ARRIVAL)) P.withhold = 1;
  if (opts && (opts->flags & MOE_OPT_WITHHOLD_H)) P.withhold_h = 1;
  if (opts && (opts->flags & MOE_OPT_TRACE))
    P.trace = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + make_layout(dims, topk).trace);
  const int grid = grid_for(di, layer_kernel(L.v, L.mm), L.lds, opts ? opts->grid : 0);
  return launch_layer(P, L, grid, (hipStream_t)stream, opts && (opts->flags & MOE_OPT_COOPERATIVE));
}

int moe_mxfp4_forward(const moe_mxfp4_dims* dims, const void* x, const float* router_w,
                      const uint8_t* packed_experts, const uint8_t* scales, int32_t topk, float* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return moe_mxfp4_forward_ex(dims, x, router_w, packed_experts, scales, topk, out, workspace, workspace_bytes,
                              nullptr, stream);
}

int moe_mxfp4_forward_noalloc(const moe_mxfp4_dims* dims, const void* x, const float* router_w,
                              const uint8_t* packed_experts, const uint8_t* scales, int32_t topk, float* out,
                              void* stream) {
  int st = check_dims(dims, topk);
  if (st != MOE_OK) return st;
  if (dims->T == 0) return MOE_OK;
  const size_t need = make_layout(dims, topk).total;
  if (need > kScratchBytes) return MOE_EWORKSPACE;
  // the pointers are checked before the scratch is set up (which may enqueue
  // its first zero fill)
  st = check_io_ptrs(x, router_w, packed_experts, scales, out);
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  st = scratch_for_device((hipStream_t)stream, &ws);
  if (st != MOE_OK) return st;
  return moe_mxfp4_forward_ex(dims, x, router_w, packed_experts, scales, topk, out, ws, need, nullptr, stream);
}

int moe_mxfp4_forward_staged(const moe_mxfp4_dims* dims, const void* x, const float* router_w,
                             const uint8_t* packed_experts, const uint8_t* scales, int32_t topk, float* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(dims, topk);
  if (st != MOE_OK) return st;
  if (dims->T == 0) return MOE_OK;
  st = check_ptrs(x, router_w, packed_experts, scales, out, workspace);
  if (st != MOE_OK) return st;
  if (workspace_bytes < make_layout(dims, topk).total) return MOE_EWORKSPACE;
  Launch L;
  st = plan_launch(dims, topk, &L);
  if (st != MOE_OK) return st;
  DeviceInfo di;
  st = device_info(&di);
  if (st != MOE_OK) return st;
  Params P = make_params(dims, topk, x, router_w, packed_experts, scales, out, workspace, di, 0u);
  apply_launch(P, L);
  return launch_staged(P, L, di.cus, (hipStream_t)stream, true);
}

int moe_mxfp4_route(const moe_mxfp4_dims* dims, const void* x, const float* router_w, int32_t topk,
                    int32_t* topk_idx, float* topk_w, int32_t* expert_offsets, int32_t* sorted_slot, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = check_dims(dims, topk);
  if (st != MOE_OK) return st;
  if (dims->T == 0) return MOE_OK;
  if (!x || !router_w || !workspace) return MOE_EINVAL;
  if ((uintptr_t)x % 16 || (uintptr_t)router_w % 16 || (uintptr_t)workspace % kAlign) return MOE_EALIGN;
  if (workspace_bytes < make_layout(dims, topk).total) return MOE_EWORKSPACE;
  Launch L;
  st = plan_launch(dims, topk, &L);
  if (st != MOE_OK) return st;
  DeviceInfo di;
  st = device_info(&di);
  if (st != MOE_OK) return st;
  // packed/scales/out are not touched by the routing kernels
  Params P = make_params(dims, topk, x, router_w, nullptr, nullptr, nullptr, workspace, di, 0u);
  apply_launch(P, L);
  hipStream_t s = (hipStream_t)stream;
  st = launch_staged(P, L, di.cus, s, false);
  if (st != MOE_OK) return st;
  const size_t TK = (size_t)dims->T * topk;
  if (topk_idx && hipMemcpyAsync(topk_idx, P.topk_idx, TK * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_EDEVICE;
  if (topk_w && hipMemcpyAsync(topk_w, P.topk_w, TK * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_EDEVICE;
  if (expert_offsets &&
      hipMemcpyAsync(expert_offsets, P.offsets, ((size_t)dims->E + 1) * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_EDEVICE;
  if (sorted_slot && hipMemcpyAsync(sorted_slot, P.sorted_slot, TK * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_EDEVICE;
  return MOE_OK;
}

int moe_mxfp4_layers_one_launch(const moe_mxfp4_dims* dims, int32_t topk) {
  int st = check_dims(dims, topk);
  if (st != MOE_OK) return -st;
  Launch L;
  st = plan_launch(dims, topk, &L);
  if (st != MOE_OK) return -st;
  return stack_kernel(L.v, L.mm) != nullptr ? 1 : 0;
}

int moe_mxfp4_forward_layers(const moe_mxfp4_dims* dims, int32_t layers, const void* x, const float* router_w,
                             const uint8_t* packed_experts, const uint8_t* scales, int32_t topk, float* out,
                             void* workspace, size_t workspace_bytes, int32_t flags, void* stream) {
  int st = check_dims(dims, topk);
  if (st != MOE_OK) return st;
  if (layers < 1 || layers > kMaxLayers) return MOE_EINVAL;
  if (flags & ~(MOE_LAYERS_PER_LAUNCH | MOE_LAYERS_ONE_LAUNCH | MOE_LAYERS_COOPERATIVE)) return MOE_EINVAL;
  if ((flags & MOE_LAYERS_PER_LAUNCH) && (flags & MOE_LAYERS_ONE_LAUNCH)) return MOE_EINVAL;
  if (dims->T == 0) return MOE_OK;
  st = check_ptrs(x, router_w, packed_experts, scales, out, workspace);
  if (st != MOE_OK) return st;
  if (workspace_bytes < make_layout(dims, topk).total) return MOE_EWORKSPACE;
  Launch L;
  st = plan_launch(dims, topk, &L);
  if (st != MOE_OK) return st;
  const void* sk = stack_kernel(L.v, L.mm);
  if ((flags & MOE_LAYERS_ONE_LAUNCH) && !sk) return MOE_ESHAPE;
  DeviceInfo di;
  st = device_info(&di);
  if (st != MOE_OK) return st;
  Params P = make_params(dims, topk, x, router_w, packed_experts, scales, out, workspace, di, 0u);
  apply_launch(P, L);
  P.stack_layers = layers;
  P.wr_stride = (size_t)dims->E * dims->d;
  P.pk_stride = (size_t)dims->E * moe_mxfp4_expert_packed_bytes(dims->d, dims->ffn);
  P.sc_stride = (size_t)dims->E * moe_mxfp4_expert_scale_bytes(dims->d, dims->ffn);
  hipStream_t s = (hipStream_t)stream;
  const bool coop = (flags & MOE_LAYERS_COOPERATIVE) != 0;
  if (flags & MOE_LAYERS_ONE_LAUNCH) {
    P.nlayers = layers;
    void* args[] = {&P};
    const int grid = grid_for(di, sk, L.lds, 0);
    const hipError_t e = coop ? hipLaunchCooperativeKernel(sk, dim3(grid), dim3(kWG), args, (unsigned)L.lds, s)
                              : hipLaunchKernel(sk, dim3(grid), dim3(kWG), args, (unsigned)L.lds, s);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return MOE_ELAUNCH;
    }
    return MOE_OK;
  }
  // one launch per operator: per layer, the normalisation of its input into
  // xb, then a lone-layer launch on xb that adds onto the stream
  const int grid = grid_for(di, layer_kernel(L.v, L.mm), L.lds, 0);
  for (int l = 0; l < layers; ++l) {
    Params Q = P;
    Q.layer0 = l;
    Q.wr = P.wr + (size_t)l * P.wr_stride;
    Q.packed = P.packed + (size_t)l * P.pk_stride;
    Q.scales = P.scales + (size_t)l * P.sc_stride;
    Q.x = P.xb;
    hipLaunchKernelGGL(k_norm, dim3(dims->T), dim3(kWG), 0, s, Q);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    st = launch_layer(Q, L, grid, s, coop);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

int moe_mxfp4_status(void* workspace, void* stream) {
  if (!workspace) return MOE_EINVAL;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOE_EDEVICE;
  uint32_t st = 0;
  uint32_t* w = reinterpret_cast<uint32_t*>(workspace) + kStatus;
  if (hipMemcpy(&st, w, 4, hipMemcpyDeviceToHost) != hipSuccess) return MOE_EDEVICE;
  const uint32_t zero = 0;
  if (hipMemcpy(w, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return MOE_EDEVICE;
  return (int)st;
}

const char* moe_mxfp4_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ESHAPE: return "unsupported shape";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_ELAUNCH: return "kernel launch failed";
    case MOE_ETIMEOUT: return "device wait timed out";
    case MOE_EDEVICE: return "device query or copy failed";
    case MOE_EALIGN: return "misaligned pointer";
    default: return "unknown status";
  }
}

}  // extern "C"
