/*
 * moe_mxfp4.h -- C ABI of the MXFP4 MoE expert layer for AMD Instinct MI355X (gfx950).
 *
 * One call runs one Mixture-of-Experts layer over a block of T tokens:
 *   router logits -> top-k experts and gates -> token-to-expert permutation
 *   -> MXFP4-dequant gate/up projections with SwiGLU -> MXFP4 down projection
 *   -> gate-weighted combine.
 * All of it runs in HIP kernels on the GPU; the host side only validates
 * arguments and enqueues work on the caller's stream.
 *
 * Sources (pages on the MiMo x TileRT system; cited by title and section):
 *  [P1-FP4]  "MiMo x TileRT" article (blog.hypho.cn), section "第一层：FP4 选择性量化":
 *            MoE expert weights are OCP MXFP4, the router keeps a higher precision.
 *  [P1-BG]   same article, section "万亿参数推理为什么特别难": each token activates a
 *            few experts and decode speed is bounded by bandwidth / bytes per token.
 *  [P3-FP4]  "MiMo 把 1T 模型推到每秒千 token——FP4、DFlash 與常駐 kernel 的三層
 *            co-design" (vatt-ghern.pages.dev), section "FP4：只量化 MoE expert，其餘
 *            維持原精度": small blocks of 4-bit values share one scale; top-k routing
 *            is precision sensitive.
 *  [P3-PK]   same page, section "persistent engine kernel 與 warp specialization":
 *            one resident kernel instead of one launch per operator.
 *  [P3-DF]   same page, section "DFlash：block-level masked 並行草稿": one target
 *            forward verifies a block of 8 drafted positions.
 *  [P5-FP4]  "tech-implementation-2026-06-09" (shengyayun.com), section "关键实现细节
 *            / 1.": the quantized linears are the experts' gate_proj, up_proj, down_proj.
 *  [P5-TRT]  same page, section "3. TileRT 的"持久化内核"到底做了什么": per layer, the
 *            MoE gate then the expert compute; per-op launches leave gaps.
 *  [MX]      OCP Microscaling Formats v1.0 (listed among the pages' sources): E2M1
 *            elements, 32-element blocks, E8M0 scales 2^(s-127).
 *
 * Data layout (all row-major; K is the contiguous, reduced dimension):
 *  x              bf16 [T][d]                               (device)
 *  router_w       fp32 [E][d]                               (device)
 *  packed_experts uint8, expert e at byte e*moe_mxfp4_expert_packed_bytes(d, F):
 *                   gate [F][d/2] | up [F][d/2] | down [d][F/2]
 *                 element c of a row is in byte c/2 of that row, low nibble for
 *                 even c, high nibble for odd c; each nibble is an E2M1 code.
 *  scales         uint8, expert e at byte e*moe_mxfp4_expert_scale_bytes(d, F):
 *                   gate [F][d/32] | up [F][d/32] | down [d][F/32]
 *                 one E8M0 byte per 32 consecutive elements of a row.
 *  out            fp32 [T][d]                               (device, overwritten)
 *
 * Semantics (readings where the pages are silent):
 *  logit[t][e] = sum_c x[t][c] * router_w[e][c], fp32 accumulation;
 *  top-k: the k largest logits of a token, ties toward the lower expert index;
 *  gate[t][j] = softmax over the k selected logits;
 *  h = silu(W_gate x_t) * (W_up x_t), y = W_down h (dequantized weights, fp32
 *  accumulation, h kept in fp32);
 *  out[t] = sum_j gate[t][j] * y(expert_j, t), summed in top-k order.
 *  Scale bytes: every byte s in 0..254 decodes as 2^(s-127), byte 0 included
 *  (2^-127, with subnormal element values kept, as measured on MI355X and
 *  checked against the fp64 oracle by the GPU tests); an element whose value
 *  exceeds the fp32 range (a large code at s = 253 or 254) decodes as +-inf.
 *  Byte 255 (NaN in the format) is not supported.
 *  h: kept in fp32 on the small-batch path; on the MFMA path (more than 48
 *  tokens whose x does not fit in LDS) the down projection takes h as the sum
 *  of two bf16 values (hi, lo), i.e. to about 16 significant bits.
 *
 * Ownership and concurrency: the caller allocates and frees every buffer.  The
 * library never allocates device memory, never synchronizes (except
 * moe_mxfp4_status) and returns as soon as the work is enqueued on `stream`
 * (a hipStream_t; NULL is the default stream).  Inputs are read-only.  A
 * workspace must not be shared by two calls that may run concurrently; its
 * contents other than the synchronization header are undefined after a call.
 *
 * Errors: every entry point returns a moe_status.  Host-side validation
 * happens before anything is enqueued; on an error nothing runs.  With T = 0
 * (valid sizes) a call does nothing and returns MOE_OK without looking at the
 * buffer pointers.  Device faults surface at the caller's next
 * synchronization, as for any HIP call.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,     /* null pointer, topk outside [1, E], negative T, bad option   */
  MOE_ESHAPE = 2,     /* d or ffn not a multiple of 32, or a size above the limits   */
  MOE_EWORKSPACE = 3, /* workspace smaller than moe_mxfp4_workspace_bytes()          */
  MOE_ELAUNCH = 4,    /* the HIP launch failed                                       */
  MOE_ETIMEOUT = 5,   /* a device-side wait exceeded its limit; the kernel exited    */
  MOE_EDEVICE = 6,    /* HIP device query / copy failed                              */
  MOE_EALIGN = 7      /* x, router_w, packed_experts or out not 16-byte aligned,
                         workspace not 256-byte aligned                              */
} moe_status;

/* Layer sizes: T tokens, hidden size d, expert ffn size, E experts.  Limits:
 * T >= 0, d and ffn multiples of 32, 32 <= d <= 8192, 32 <= ffn <= 4096, 1 <= E <= 1024,
 * E * ceil(T / 64) <= 4096 (so T <= 1024 with 256 experts), 1 <= topk <= min(E, 64). */
typedef struct {
  int32_t T;
  int32_t d;
  int32_t ffn;
  int32_t E;
} moe_mxfp4_dims;

/* Bytes of one expert's packed codes: 3*d*ffn/2 ([P5-FP4] three linears per expert). */
size_t moe_mxfp4_expert_packed_bytes(int32_t d, int32_t ffn);

/* Bytes of one expert's E8M0 scales: 3*d*ffn/32 ([P3-FP4] one scale per block). */
size_t moe_mxfp4_expert_scale_bytes(int32_t d, int32_t ffn);

/* Size of the device workspace moe_mxfp4_forward needs for these sizes (0 on
 * invalid sizes).  It holds a synchronization header, the router's partial
 * logits, the top-k results, the SwiGLU activations h [T*topk][ffn] and the
 * gated expert outputs [T*topk][d] as epoch-tagged 64-bit words, and plain
 * copies of the routing results for inspection. */
size_t moe_mxfp4_workspace_bytes(const moe_mxfp4_dims* dims, int32_t topk);

/* Zero a whole workspace on `stream` (a fill kernel, safe under stream
 * capture).  A workspace must be zero-filled before its first forward call
 * (allocating it zeroed is enough); afterwards every call leaves it valid for
 * the next one.  Call it again after a forward call that timed out. */
int moe_mxfp4_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* The whole layer in ONE persistent kernel launch ([P3-PK], [P5-TRT]): router,
 * top-k, permutation, expert gate/up+SwiGLU, down projection and combine.
 * The grid is one workgroup per CU, all co-resident (see MOE_OPT_COOPERATIVE);
 * the steps hand data to each other through epoch-tagged words that consumers
 * poll, so no host round trip, grid barrier or device-wide atomic separates
 * them.  The MoE gate is [P1-FP4]/[P3-FP4]'s higher-precision router; the
 * experts are [P5-FP4]'s MXFP4 gate/up/down.
 *   dims            sizes (host pointer)
 *   x               bf16 [T][d] device, 16-byte aligned
 *   router_w        fp32 [E][d] device, 16-byte aligned
 *   packed_experts  E2M1 codes, layout above, device, 16-byte aligned
 *   scales          E8M0 bytes, layout above, device
 *   topk            experts per token, 1 <= topk <= min(E, 64)
 *   out             fp32 [T][d] device, 16-byte aligned, fully overwritten
 *   workspace       device, 256-byte aligned, >= moe_mxfp4_workspace_bytes(),
 *                   zero-filled before its first use
 *   stream          hipStream_t
 * Returns MOE_OK once enqueued.  Every device-side wait on another
 * workgroup's results has a watchdog (2 s); a wait that does not finish makes
 * the kernel exit early and sets the status word that moe_mxfp4_status()
 * returns as MOE_ETIMEOUT.  The out elements such a call could not complete
 * are then NaN (each wave whose wait was abandoned writes NaN into all of the
 * elements it combines), so out never keeps an earlier call's values; the
 * others hold this call's results. */
int moe_mxfp4_forward(const moe_mxfp4_dims* dims, const void* x, const float* router_w,
                      const uint8_t* packed_experts, const uint8_t* scales, int32_t topk,
                      float* out, void* workspace, size_t workspace_bytes, void* stream);

/* The layer without a caller workspace and without any allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments as
 * moe_mxfp4_forward minus the workspace, the same kernels and the same result
 * bit for bit.  The workspace is a 32 MiB array in the library's device
 * memory, one per GPU the library runs on, held until the process ends; its
 * address is looked up once per device, and the first call on a device
 * enqueues a zero fill of it (a kernel) on `stream` before the layer.
 * Sizes whose workspace (moe_mxfp4_workspace_bytes) exceeds 32 MiB are
 * rejected with MOE_EWORKSPACE: e.g. every T <= 32 at d = 7168, ffn = 2048,
 * E = 256, top-8 fits, T = 64 does not.  Every call on a GPU shares that GPU's
 * array: calls that may overlap on one GPU (two streams, two threads) race and
 * must not be made.  A timed-out call leaves NaN in out as moe_mxfp4_forward
 * does (its status word is not readable: there is no workspace pointer).
 * Errors: as moe_mxfp4_forward (no workspace arguments to check). */
int moe_mxfp4_forward_noalloc(const moe_mxfp4_dims* dims, const void* x, const float* router_w,
                              const uint8_t* packed_experts, const uint8_t* scales, int32_t topk, float* out,
                              void* stream);

/* Same layer and the same result bit for bit, as one kernel launch per step
 * ([P5-TRT]'s per-operator model), for measuring what the single launch saves. */
int moe_mxfp4_forward_staged(const moe_mxfp4_dims* dims, const void* x, const float* router_w,
                             const uint8_t* packed_experts, const uint8_t* scales, int32_t topk,
                             float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Options of moe_mxfp4_forward_ex. */
typedef struct {
  uint32_t flags;         /* MOE_OPT_* bits                                           */
  uint32_t spin_limit_us; /* device wait limit in microseconds; 0 = default (2 s)      */
  int32_t grid;           /* workgroups of the persistent launch; 0 = all co-resident  */
} moe_mxfp4_options;

/* Test knob: the top-k step waits for router results tagged for a call that
 * never happens, so every workgroup reaches its watchdog and the kernel exits
 * with MOE_ETIMEOUT. */
#define MOE_OPT_WITHHOLD_ARRIVAL 0x1u

/* Step trace: the first wave of every workgroup of the persistent launch
 * writes the device wall clock (hipDeviceAttributeWallClockRate kHz) when it
 * ends each step, into the workspace's trace region (offset `trace` of
 * moe_mxfp4_ws_layout): uint64 [grid][16], slots 0 start, 1 router (and x
 * staged), 7 own top-k tokens published, 2 all top-k results read,
 * 3 permutation, 4 gate/up, 8 first h needed by the down step present,
 * 5 down, 6 combine; 9-15 the gate/up end of waves 1-7 (slot 4 is wave 0's).
 * Costs one store per step and workgroup. */
#define MOE_OPT_TRACE 0x2u

/* Launch the persistent kernel cooperatively (hipLaunchCooperativeKernel):
 * the runtime then guarantees that all its workgroups are resident at once.
 * By default the kernel is launched normally, which on MI355X saves ~17 us per
 * call; its grid (one workgroup per CU, each filling its CU) is then resident
 * at once as long as no other kernel holds CUs, and if one does, the layer's
 * waits end with MOE_ETIMEOUT instead of hanging. */
#define MOE_OPT_COOPERATIVE 0x4u

/* Test knob: the down step waits for h words tagged for a call that never
 * happens, so every down wait reaches its watchdog; the call ends with
 * MOE_ETIMEOUT and every element of out NaN. */
#define MOE_OPT_WITHHOLD_H 0x8u

/* moe_mxfp4_forward with options (opts may be NULL). */
int moe_mxfp4_forward_ex(const moe_mxfp4_dims* dims, const void* x, const float* router_w,
                         const uint8_t* packed_experts, const uint8_t* scales, int32_t topk,
                         float* out, void* workspace, size_t workspace_bytes,
                         const moe_mxfp4_options* opts, void* stream);

/* Routing only ([P1-BG] each token to a few experts; [P3-FP4] top-k): runs the
 * router, top-k and permutation kernels of the layer and copies their results
 * (device buffers):
 *   topk_idx       int32 [T][topk]  experts of each token, (logit desc, index asc)
 *   topk_w         fp32  [T][topk]  gates
 *   expert_offsets int32 [E+1]      pairs routed to experts < e
 *   sorted_slot    int32 [T*topk]   pair p's slot t*topk + j; pairs ordered by
 *                                   (expert asc, token asc)
 * Any output pointer may be NULL.  Same validation as moe_mxfp4_forward. */
int moe_mxfp4_route(const moe_mxfp4_dims* dims, const void* x, const float* router_w, int32_t topk,
                    int32_t* topk_idx, float* topk_w, int32_t* expert_offsets, int32_t* sorted_slot,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Byte offsets of the intermediates inside a workspace after a forward call
 * (for inspection).  h = SwiGLU activations [T*topk][ffn] in pair order (the
 * order of sorted_slot; within a pair's row the values are in order when
 * h_chunk_major is 0, else value i = 32 c + e is word 2 ((e / 2) (ffn / 32) + c)
 * + e % 2 of the row, the order the small-batch path with x of every token in
 * LDS reads in its down step) and
 * y = gated expert outputs [T*topk][d] in slot order
 * (row t*topk + j holds gate[t][j] * y(expert_j, t)) are 64-bit words whose low
 * 32 bits are the fp32 value (the high 32 bits are a tag); logits fp32 [T][E];
 * topk_idx int32 [T][topk]; topk_w fp32 [T][topk]; offsets int32 [E+1];
 * sorted_slot, pos int32 [T*topk]; active int32 [E] (experts with at least one
 * token, ascending); n_active int32; trace: see MOE_OPT_TRACE; x_last bf16
 * [T][d], after a stack call (moe_mxfp4_forward_layers) the normalised input
 * of its last layer. */
typedef struct {
  size_t logits, topk_idx, topk_w, offsets, sorted_slot, pos, active, n_active, h, y, trace, x_last, h_chunk_major,
      total;
} moe_mxfp4_ws_layout;
int moe_mxfp4_workspace_layout(const moe_mxfp4_dims* dims, int32_t topk, moe_mxfp4_ws_layout* layout);

/* Wait for `stream`, then read and clear the workspace's device status word:
 * MOE_OK, or MOE_ETIMEOUT if a device wait of the last call(s) timed out. */
int moe_mxfp4_status(void* workspace, void* stream);

/* Static description of a status code. */
const char* moe_mxfp4_strerror(int status);

/* Grid (workgroups) the persistent launch uses on the current device for these
 * sizes, or a negative moe_status. */
int moe_mxfp4_persistent_grid(const moe_mxfp4_dims* dims, int32_t topk);

/* ---- A stack of layers on one residual stream ([P5-TRT]: the resident
 * engine runs the model layer after layer, each layer's MoE gate then its
 * expert compute; [P3-PK]: the pipeline stays on the GPU between operators,
 * whose per-operator model lists the normalisation among them).  Reading (the
 * pages describe the MoE layer alone): a pre-norm residual block without its
 * attention, the normalisation with unit gain (no trained weights):
 *   r_0 = x;  x_l = bf16(r_l / sqrt(mean over d of r_l^2 + 1e-6)) (fp32
 *   arithmetic, round to nearest even);
 *   r_{l+1} = r_l + MoE_l(x_l) (fp32);  out = r_L.
 *   dims, topk      as for moe_mxfp4_forward, the same for every layer
 *   layers          L, 1 <= L <= 4096
 *   x               bf16 [T][d], the stack's input (device, 16-byte aligned)
 *   router_w        fp32 [L][E][d] (device, 16-byte aligned)
 *   packed_experts  [L] x the layer's E experts, layer l at byte
 *                   l*E*moe_mxfp4_expert_packed_bytes(d, F) (device, 16-byte aligned)
 *   scales          [L] x the layer's E experts, layer l at byte
 *                   l*E*moe_mxfp4_expert_scale_bytes(d, F) (device)
 *   out             fp32 [T][d] = r_L (device, 16-byte aligned, fully
 *                   overwritten; it holds intermediate r_l while the stack
 *                   runs, so it must not overlap any input)
 *   workspace       as for moe_mxfp4_forward (same size).  After the call its
 *                   inspection copies describe the last layer, and x_last
 *                   (moe_mxfp4_ws_layout) holds that layer's input.
 *   flags           0 or MOE_LAYERS_PER_LAUNCH: one launch per operator (per
 *                   layer: the normalisation, then the layer);
 *                   MOE_LAYERS_ONE_LAUNCH: the whole stack in ONE resident
 *                   launch, for sizes on the small-batch path with x of every
 *                   token in LDS (moe_mxfp4_layers_one_launch), else
 *                   MOE_ESHAPE.  Measured on MI355X (8 verify-block layers):
 *                   one launch per operator ~250 us per layer, one resident
 *                   launch ~268 us: back-to-back launches from one stream leave
 *                   no measurable gap, so the default is the per-operator one.
 * In the one launch, the workgroups meet between layers: each publishes its
 * part of the stream and raises an arrival word; once every arrival word has
 * moved on, each workgroup normalises the stream into its LDS and the next
 * layer's router starts (its first weight loads are issued before the wait).  Errors as moe_mxfp4_forward, and
 * MOE_EINVAL for L out of range or unknown / conflicting flags.  A device
 * wait that times out stops the stack (MOE_ETIMEOUT from moe_mxfp4_status);
 * the elements of out it could not complete are then NaN, as for
 * moe_mxfp4_forward (in the one-launch mode every element a stopped
 * workgroup combines). */
#define MOE_LAYERS_PER_LAUNCH 0x1
#define MOE_LAYERS_ONE_LAUNCH 0x2
/* Either mode, launched cooperatively (see MOE_OPT_COOPERATIVE): the runtime
 * then guarantees that each launch's workgroups are resident at once. */
#define MOE_LAYERS_COOPERATIVE 0x4
int moe_mxfp4_forward_layers(const moe_mxfp4_dims* dims, int32_t layers, const void* x, const float* router_w,
                             const uint8_t* packed_experts, const uint8_t* scales, int32_t topk, float* out,
                             void* workspace, size_t workspace_bytes, int32_t flags, void* stream);

/* 1 if moe_mxfp4_forward_layers can run these sizes as one resident launch
 * (MOE_LAYERS_ONE_LAUNCH), 0 if not, or a negative moe_status. */
int moe_mxfp4_layers_one_launch(const moe_mxfp4_dims* dims, int32_t topk);

/* ---- MXFP4 quantize / pack on the GPU ([P3-FP4] 4-bit values with a shared
 * per-block scale; [MX] conversion): the direction opposite to the layer's
 * decode, to prepare expert weights in the layout above on the device.
 *
 *   w       rows x K values, row-major, device; fp32 (dtype MOE_QDTYPE_F32) or
 *           bf16 bit patterns (MOE_QDTYPE_BF16); 16-byte aligned; finite.
 *   packed  rows x K/2 bytes (device, 4-byte aligned, overwritten): element c
 *           of a row in byte c/2, low nibble for even c.
 *   scales  rows x K/32 bytes (device, overwritten): the E8M0 byte of each
 *           32-element block.
 * Rule per block: X = floor(log2 max|v|) - 2 clamped to [-127, 127] (-127 for
 * an all-zero block), scale byte X + 127; each element to the E2M1 magnitude
 * nearest |v| / 2^X, ties to the even mantissa bit, saturating at 6; sign bit
 * when v < 0.  Non-finite inputs give unspecified codes.
 * Errors: MOE_EINVAL (null pointer, negative size, unknown dtype), MOE_ESHAPE
 * (K not a multiple of 32), MOE_EALIGN, MOE_EDEVICE, MOE_ELAUNCH.  rows = 0 or
 * K = 0 does nothing.  Enqueued on `stream`; nothing is allocated. */
enum { MOE_QDTYPE_F32 = 0, MOE_QDTYPE_BF16 = 1 };
int moe_mxfp4_quantize(const void* w, int32_t dtype, int64_t rows, int64_t K, uint8_t* packed, uint8_t* scales,
                       void* stream);

/* ---- MXFP4 codec on the host ([P3-FP4] "FP4：只量化 MoE expert，其餘維持原精度":
 * each small block of weights is stored as 4-bit values plus one shared
 * scale; [MX] E2M1 elements, 32-element blocks, E8M0 scales 2^(s-127)).  Host
 * memory only; nothing is enqueued and no GPU is needed.
 *
 * moe_mxfp4_quantize_host: rows x K fp32 values (row-major, host) -> packed
 * [rows][K/2] codes (element c of a row in byte c/2, low nibble for even c)
 * and scales [rows][K/32] E8M0 bytes, by the rule of moe_mxfp4_quantize
 * (X = floor(log2 max|v|) - 2 clamped to [-127, 127], -127 for an all-zero
 * block; nearest E2M1 magnitude of |v| / 2^X, ties to the even mantissa bit,
 * saturating at 6; sign bit when v < 0, so -0 gives code 0).
 * moe_mxfp4_dequantize_host: the reverse, value = E2M1(code) * 2^(s-127)
 * rounded to fp32: exact whenever the product is an fp32 value (every code at
 * s <= 252), +-inf where it exceeds the fp32 range (large codes at s = 253,
 * 254), NaN for s = 255.
 * Errors: MOE_EINVAL (null pointer with rows, K > 0; negative size; a
 * non-finite input value to quantize, checked before anything is written),
 * MOE_ESHAPE (K not a multiple of 32).  rows = 0 or K = 0 does nothing.  The
 * caller owns every buffer. */
int moe_mxfp4_quantize_host(const float* w, int64_t rows, int64_t K, uint8_t* packed, uint8_t* scales);
int moe_mxfp4_dequantize_host(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t K, float* w);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
