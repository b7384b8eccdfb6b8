/*
 * mxfp4_moe.h -- C ABI of the MXFP4 routed-expert MoE layer for MI355X (gfx950).
 *
 * The layer (one GPU's share of it):
 *   1. route:    per token, softmax over the E_global router logits, the top_k
 *                experts, weights renormalised over those k picks;
 *   2. permute:  the (token, slot) assignments whose expert is local
 *                (first_local <= id < first_local + E_local) are counted per
 *                expert, prefix-summed and scattered into expert-contiguous order,
 *                keeping (token, slot) order inside each expert;
 *   3. gate_up:  per assignment, h = W13_e x_t  (W13_e = [gate | up], 2I x H);
 *   4. SwiGLU:   a = bf16( silu(min(g, L)) * clamp(u, -L, L) );
 *   5. down:     y = W2_e a  (W2_e: H x I);
 *   6. combine:  out[t] = bf16( sum over the token's local slots of w * y ).
 * Weights are MXFP4: E2M1 codes, two per byte, and one UE8M0 power-of-two scale
 * per 32 consecutive elements along K.
 *
 * Sources: the element format and its fixed 16-entry codebook and the OCP
 * Microscaling block scale -- XFP blog, section "路线二：硬件格式（NVFP4 / MXFP4）";
 * packed storage (a packed row is half the logical width) with a separate scale
 * tensor, and a fused per-layer buffer of all experts -- campaign page
 * "glm53-mxfp4-mi355x", sections "A fused tensor with two dtypes in it" and "The
 * model card and the metadata disagree"; per-token reads of only the routed
 * experts -- same page, section "A file is a census; a decode step is a sample";
 * [gate | up] stacked into one weight feeding the SwiGLU -- TensorFold PR #1050,
 * commit notes; the clamp kept by the MI355X experts -- model card
 * "GLM-5.3-Flash-MXFP4", section "Verification compute and EAGLE"; refusing
 * empty or overflowing shapes by name with checked arithmetic -- TensorFold PR
 * #1050, review and commit notes.
 *
 * Conventions for every entry point:
 *   - Status: 0 = MXFP4_MOE_OK, negative = a named refusal (see
 *     mxfp4_moe_status_string).  All argument checks run on the host before any
 *     GPU work is enqueued, so a refused call has enqueued nothing.
 *   - Memory: every tensor pointer is device memory owned by the caller, 16-byte
 *     aligned.  The library allocates nothing.  Inputs are read-only; outputs are
 *     fully overwritten; the workspace's contents are undefined afterwards.
 *   - Execution: work is enqueued on `stream` (0 = the null stream) and the call
 *     returns without waiting.  Calls on different streams with different
 *     workspaces may run concurrently.  The only process-wide state is a set of
 *     per-device caches filled once under a lock (the device check, the CU
 *     count, resident-grid sizes, kernels' LDS limits) and the static scratch of
 *     mxfp4_moe_forward_noalloc; results never depend on it.  The library reads
 *     no environment variables.  A forward enqueues kernels only (no memset or
 *     copy nodes, no host synchronisation), so it can be recorded into a HIP
 *     graph and replayed.
 *   - Shapes: int64 counts, validated with checked arithmetic.  H and I must be
 *     multiples of 128; T may be 0 (nothing is enqueued).
 *   - Preconditions not checked (for cost): router logits are not NaN (a NaN
 *     logit gives an unspecified routing); NaN/inf in x or weights propagate.
 */
#ifndef MXFP4_MOE_H
#define MXFP4_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXFP4_MOE_ABI_VERSION 1

/* status codes */
#define MXFP4_MOE_OK 0
#define MXFP4_MOE_ERR_NULL_POINTER (-1)        /* a required pointer is NULL */
#define MXFP4_MOE_ERR_EMPTY_SHAPE (-2)         /* H, I, E_global, E_local or top_k is 0 */
#define MXFP4_MOE_ERR_SHAPE_OVERFLOW (-3)      /* a byte or element count overflows */
#define MXFP4_MOE_ERR_UNSUPPORTED_SHAPE (-4)   /* H or I not a multiple of 128, negative
                                                  sizes, E_global > 512, or local range
                                                  outside E_global */
#define MXFP4_MOE_ERR_BAD_TOP_K (-5)           /* top_k < 1, > E_global or > 32 */
#define MXFP4_MOE_ERR_BAD_CLAMP (-6)           /* clamp_limit NaN or <= 0 (+inf = no clamp) */
#define MXFP4_MOE_ERR_WORKSPACE_TOO_SMALL (-7) /* workspace_bytes below the required size */
#define MXFP4_MOE_ERR_MISALIGNED (-8)          /* a device pointer is not 16-byte aligned */
#define MXFP4_MOE_ERR_UNSUPPORTED_DEVICE (-9)  /* current device is not gfx950 / no device */
#define MXFP4_MOE_ERR_HIP (-10)                /* a HIP call failed (see last_hip_error) */
#define MXFP4_MOE_ERR_BAD_FLAGS (-11)          /* unknown flag bits */
#define MXFP4_MOE_ERR_BAD_ARGUMENT (-12)       /* any other invalid scalar argument */
#define MXFP4_MOE_ERR_SCRATCH_LIMIT (-13)      /* mxfp4_moe_forward_noalloc: the call needs more
                                                  workspace than its static scratch holds */

/* flags */
#define MXFP4_MOE_A4 0x1u            /* quantise x (along H) and the SwiGLU output (along
                                        I) to MXFP4 with the OCP rule and run both
                                        contractions on scaled FP4 MFMA */
#define MXFP4_MOE_DETERMINISTIC 0x2u /* combine by an ordered gather instead of fp32
                                        atomics: bit-identical results run to run */
#define MXFP4_MOE_SHARED_EXPERT 0x4u /* the weight buffers hold E_local + 1 experts: the
                                        last is a shared MXFP4 expert of the same shape
                                        that every token reads with weight 1 (the
                                        always-active MoE MLP whose projections the
                                        campaign page "glm53-mxfp4-mi355x", section "The
                                        model card and the metadata disagree", finds
                                        stored as packed FP4 with a scale tensor).  It
                                        takes one more slot per token, after the top_k
                                        routed ones: routing tables and intermediates
                                        below then have top_k + 1 slots per token and
                                        E_local + 1 experts (slot top_k: id E_global,
                                        weight 1, table expert E_local).  In an
                                        expert-parallel split exactly one share sets it. */
#define MXFP4_MOE_A8 0x8u            /* as MXFP4_MOE_A4 with MXFP8 activations: E4M3
                                        elements (one byte each) under the same UE8M0
                                        block scale (mxfp4_moe_quantize8), the FP8
                                        operand of the same scaled MFMA.  Excludes
                                        MXFP4_MOE_A4 (both: BAD_FLAGS).  Intermediates
                                        below then hold one code byte per element. */
#define MXFP4_MOE_ROUTE_LAUNCH 0x10u /* route in a launch of its own even where the
                                        gate_up kernel would route the tokens itself
                                        (few tokens): same tables and results, one
                                        launch more; lets a caller compare the forms */

typedef struct mxfp4_moe_dims {
  int64_t T;           /* tokens */
  int64_t H;           /* hidden size (K of gate_up, N of down) */
  int64_t I;           /* per-expert intermediate size */
  int64_t E_global;    /* experts the router chooses among (logit columns) */
  int64_t E_local;     /* experts held by this GPU */
  int64_t first_local; /* global id of local expert 0 */
  uint32_t flags;      /* MXFP4_MOE_A4 or MXFP4_MOE_A8, | MXFP4_MOE_DETERMINISTIC
                          | MXFP4_MOE_SHARED_EXPERT | MXFP4_MOE_ROUTE_LAUNCH */
  uint32_t reserved;   /* must be 0 */
} mxfp4_moe_dims;

/* ABI version (MXFP4_MOE_ABI_VERSION of the built library). */
int mxfp4_moe_abi_version(void);

/* Static name of a status code ("MXFP4_MOE_OK", "MXFP4_MOE_ERR_..."); never NULL. */
const char* mxfp4_moe_status_string(int status);

/* hipError_t of the most recent MXFP4_MOE_ERR_HIP returned on the calling thread. */
int mxfp4_moe_last_hip_error(void);

/*
 * Sizes of the preshuffled (gfx950) weight tensors for all E_local experts (and
 * the shared one with MXFP4_MOE_SHARED_EXPERT).
 * Outputs: bytes of w13 codes, w13 scales, w2 codes, w2 scales.  Codes keep the
 * canonical byte count; scales are padded to whole 512-element K groups.
 */
int mxfp4_moe_preshuffled_bytes(const mxfp4_moe_dims* d, size_t* w13_bytes,
                                size_t* w13_scale_bytes, size_t* w2_bytes, size_t* w2_scale_bytes);

/*
 * One-time weight layout change, canonical -> gfx950 preshuffled.
 * Canonical inputs (device; E_local + 1 experts with MXFP4_MOE_SHARED_EXPERT,
 * the shared one last):
 *   canon_w13  uint8 [E_local][2I][H/2]   rows 0..I-1 gate, I..2I-1 up; element k of
 *                                          a row in byte k/2, low nibble for even k
 *   canon_w13s uint8 [E_local][2I][H/32]  UE8M0 scale of elements 32b..32b+31
 *   canon_w2   uint8 [E_local][H][I/2],  canon_w2s uint8 [E_local][H][I/32]
 * Outputs: buffers of the sizes mxfp4_moe_preshuffled_bytes reports.  The layout
 * puts the 32 elements of one MX block of one row in one 16-byte lane load, with
 * gate and up row groups interleaved.  It is an implementation detail: treat the
 * preshuffled tensors as opaque and feed them only to mxfp4_moe_forward*.
 */
int mxfp4_moe_preshuffle(const mxfp4_moe_dims* d, const uint8_t* canon_w13,
                         const uint8_t* canon_w13s, const uint8_t* canon_w2,
                         const uint8_t* canon_w2s, uint8_t* w13, uint8_t* w13s, uint8_t* w2,
                         uint8_t* w2s, hipStream_t stream);

/*
 * Load-time weight conversion in one pass: unquantised expert weights ->
 * the preshuffled MXFP4 tensors of mxfp4_moe_preshuffle, with no canonical
 * intermediate.  The conversion packs 4-bit values with a shared block scale
 * per expert tensor (campaign page "glm53-mxfp4-mi355x", section "The
 * baseline is already one byte, and the exclusions are two") and is paid once,
 * at load time, not per step (XFP blog, section "编码成本").
 * Inputs (device, in_dtype MXFP4_MOE_DTYPE_F32 or _BF16; E_local + 1 experts
 * with MXFP4_MOE_SHARED_EXPERT): w13 [E_local][2I][H] (rows 0..I-1 gate,
 * I..2I-1 up), w2 [E_local][H][I].  Each 32-element block along K is quantised
 * by the rule of mxfp4_moe_quantize.  Outputs: as mxfp4_moe_preshuffle's
 * (sizes from mxfp4_moe_preshuffled_bytes; the scale padding to whole
 * 512-element K groups is written as zeros).  Byte-identical to
 * mxfp4_moe_quantize per expert followed by mxfp4_moe_preshuffle.
 * Errors: as mxfp4_moe_preshuffle, BAD_ARGUMENT for another in_dtype.
 */
int mxfp4_moe_quantize_preshuffle(const mxfp4_moe_dims* d, const void* w13, const void* w2,
                                  int32_t in_dtype, uint8_t* w13_out, uint8_t* w13s_out,
                                  uint8_t* w2_out, uint8_t* w2s_out, hipStream_t stream);

/* Workspace bytes mxfp4_moe_forward / mxfp4_moe_route need for these dims and top_k. */
int mxfp4_moe_workspace_bytes(const mxfp4_moe_dims* d, int32_t top_k, size_t* bytes);

/*
 * How mxfp4_moe_forward will run these dims and top_k (a pure host query):
 * *tile_rows = token rows per gate_up tile (16: K split across waves, for
 * decode-sized calls; 64; 128: LDS-staged large tiles; 320: with MXFP4
 * activations, one tile per expert of up to 320 rows, down then on 128-row
 * tiles); *ordered_combine = 1 when the combine gathers slot-ordered y rows
 * (deterministic), 0 when it adds into an fp32 buffer with atomics.  The
 * large-tile plans always gather.
 * Errors as mxfp4_moe_workspace_bytes; NULL outputs -> NULL_POINTER.
 */
int mxfp4_moe_plan(const mxfp4_moe_dims* d, int32_t top_k, int32_t* tile_rows, int32_t* ordered_combine);

/*
 * The layer.  x: bf16 [T][H]; router_logits: float [T][E_global]; weights from
 * mxfp4_moe_preshuffle; out: bf16 [T][H] (tokens with no local assignment get
 * +0).  clamp_limit: L > 0 or +inf.  When T == 0, x, router_logits and out may
 * be NULL and nothing is enqueued.
 */
int mxfp4_moe_forward(const mxfp4_moe_dims* d, const void* x, const float* router_logits,
                      const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2,
                      const uint8_t* w2s, int32_t top_k, float clamp_limit, void* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mxfp4_moe_forward for callers that cannot allocate or pass device memory
 * beyond the layer's own tensors (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): no workspace argument.  Its
 * workspace is a static device array of MXFP4_MOE_NOALLOC_SCRATCH_BYTES inside
 * the library, one per GPU, created when the library's code is loaded on that
 * GPU and held until the process ends; its device address is looked up on the
 * first call on each device.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).
 * Arguments, results and errors as mxfp4_moe_forward, plus
 * MXFP4_MOE_ERR_SCRATCH_LIMIT when mxfp4_moe_workspace_bytes for these dims
 * and top_k exceeds MXFP4_MOE_NOALLOC_SCRATCH_BYTES (checked before any GPU
 * work; decode, verify and expert-parallel-share shapes fit, large prefill
 * chunks do not).  Every call on one GPU uses that GPU's one array: calls
 * that overlap on one GPU (other streams, other host threads) race and must
 * be ordered by the caller.  The array keeps the last call's contents; the
 * layer clears what it needs cleared itself.
 */
#define MXFP4_MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int mxfp4_moe_forward_noalloc(const mxfp4_moe_dims* d, const void* x, const float* router_logits,
                              const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2,
                              const uint8_t* w2s, int32_t top_k, float clamp_limit, void* out,
                              hipStream_t stream);

/*
 * mxfp4_moe_forward that also copies the intermediates out, in canonical order
 * (row p = sorted position p; rows at or past the assignment count are undefined):
 *   act  bf16 [T*top_k][I]        SwiGLU output (required)
 *   actq uint8 [T*top_k][I/2], acts uint8 [T*top_k][I/32]   A4 only (else may be NULL)
 *   xq   uint8 [T][H/2],      xs   uint8 [T][H/32]          A4 only (else may be NULL)
 *   out32 float [T][H]        the layer output before its bf16 rounding (may be NULL)
 */
int mxfp4_moe_forward_debug(const mxfp4_moe_dims* d, const void* x, const float* router_logits,
                            const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2,
                            const uint8_t* w2s, int32_t top_k, float clamp_limit, void* out,
                            void* workspace, size_t workspace_bytes, void* act, uint8_t* actq,
                            uint8_t* acts, uint8_t* xq, uint8_t* xs, float* out32,
                            hipStream_t stream);

/*
 * mxfp4_moe_forward that also records five caller-created events on `stream`
 * around its phases, for timing: events[0] before routing, events[1] after
 * routing (and, A4, the x quantisation), events[2] after gate_up + SwiGLU (and,
 * A4, the SwiGLU quantisation), events[3] after down + combine, events[4] after
 * the output cast (or ordered combine).  The computation is that of
 * mxfp4_moe_forward.
 */
int mxfp4_moe_forward_timed(const mxfp4_moe_dims* d, const void* x, const float* router_logits,
                            const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2,
                            const uint8_t* w2s, int32_t top_k, float clamp_limit, void* out,
                            void* workspace, size_t workspace_bytes, hipEvent_t* events,
                            hipStream_t stream);

/*
 * Routing tables only (steps 1-2).  Outputs (device):
 *   ids int32 [T][top_k] (rank order), weights float [T][top_k],
 *   counts int32 [E_local], offsets int32 [E_local+1] (offsets[E_local] = N_assign),
 *   sorted int32 [T*top_k] (first N_assign entries valid: slot t*top_k+j),
 *   inv int32 [T*top_k] (sorted position of each slot, -1 if not local).
 */
int mxfp4_moe_route(const mxfp4_moe_dims* d, const float* router_logits, int32_t top_k,
                    int32_t* ids, float* weights, int32_t* counts, int32_t* offsets,
                    int32_t* sorted, int32_t* inv, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * OCP MX quantiser: rows x K values (K % 32 == 0) -> canonical MXFP4
 * (codes uint8 [rows][K/2], scales uint8 [rows][K/32]).  Per 32-block: scale
 * byte = clamp(floor(log2 amax) - 2 + 127, 0, 254); element = E2M1 nearest to
 * v / 2^(scale-127), ties to the even code, saturating at +-6; a block holding
 * NaN or inf gets scale 0xFF and zero codes.  in_dtype: 0 = bf16, 1 = float.
 * This is the quantiser the A4 path applies to x and to the SwiGLU output, and
 * the load-time weight quantiser.
 */
#define MXFP4_MOE_DTYPE_BF16 0
#define MXFP4_MOE_DTYPE_F32 1
int mxfp4_moe_quantize(const void* in, int32_t in_dtype, int64_t rows, int64_t K, uint8_t* codes,
                       uint8_t* scales, hipStream_t stream);

/*
 * OCP MX quantiser with FP8 E4M3 elements (MXFP8; the format TensorFold PR
 * #1050's FP4-Local checkpoint stores projections in, commit notes): rows x K
 * values (K % 32 == 0) -> codes uint8 [rows][K] (one E4M3 byte per element:
 * sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7F/0xFF are NaN, no
 * infinity), scales uint8 [rows][K/32].  Per 32-block: scale byte =
 * clamp(floor(log2 amax) - 8 + 127, 0, 254); element = E4M3 nearest to
 * v / 2^(scale-127), ties to the even code, saturating at +-448; NaN/inf
 * blocks get scale 0xFF and zero codes.  Arguments and errors as
 * mxfp4_moe_quantize.  The MXFP4_MOE_A8 path applies it to x and to the SwiGLU
 * output.
 */
int mxfp4_moe_quantize8(const void* in, int32_t in_dtype, int64_t rows, int64_t K, uint8_t* codes,
                        uint8_t* scales, hipStream_t stream);

/*
 * Per-expert bf16 exclusions.  A fused expert buffer may hold packed MXFP4
 * experts and experts that were excluded from quantisation and kept in bf16;
 * a packed row is half the logical width in bytes while a bf16 row keeps it,
 * so one stride cannot slice the buffer and the exclusion set is carried per
 * expert (campaign page "glm53-mxfp4-mi355x", section "A fused tensor with two
 * dtypes in it").  E_w = E_local (+ 1 with MXFP4_MOE_SHARED_EXPERT) experts.
 *
 * Fused layout of one matrix with R rows and K columns per expert (w13: R = 2I,
 * K = H; w2: R = H, K = I): experts 0 .. E_w-1 back to back, expert e taking
 * R*K/2 bytes of canonical packed E2M1 codes ([R][K/2], as for
 * mxfp4_moe_preshuffle) when packed, or R*K*2 bytes of bf16 ([R][K]) when
 * excluded.  Its scale tensor holds R*K/32 bytes per packed expert ([R][K/32]),
 * back to back in expert order; excluded experts have none.
 */
typedef struct mxfp4_moe_bf16_experts {
  int64_t n;                  /* experts kept in bf16, 0 .. E_w (0: none, as mxfp4_moe_forward) */
  const int32_t* expert_map;  /* device int32 [E_w + n]: entry e = bf16 slot of expert e or -1;
                                 entry E_w + j = the expert in slot j (as written by
                                 mxfp4_moe_preshuffle_fused) */
  const void* w13;            /* device bf16 [n][2I][H], slot j = j-th excluded expert */
  const void* w2;             /* device bf16 [n][H][I] */
} mxfp4_moe_bf16_experts;

/*
 * Loader for a fused buffer with exclusions.  excluded: HOST uint8 [E_w], 1 =
 * kept in bf16, 0 = packed (other values: BAD_ARGUMENT); E_w <= 544.
 * Inputs (device, fused layout above): w13_fused, w13s_fused, w2_fused,
 * w2s_fused (the scale tensors may be NULL when every expert is excluded).
 * Outputs (device): w13/w13s/w2/w2s preshuffled as by mxfp4_moe_preshuffle
 * (sizes from mxfp4_moe_preshuffled_bytes; the slots of excluded experts are
 * left unwritten and never read), w13_bf16 [n][2I][H] and w2_bf16 [n][H][I]
 * (may be NULL when n = 0), expert_map int32 [E_w + n].  Enqueued on stream,
 * no host wait.
 */
int mxfp4_moe_preshuffle_fused(const mxfp4_moe_dims* d, const uint8_t* excluded,
                               const uint8_t* w13_fused, const uint8_t* w13s_fused,
                               const uint8_t* w2_fused, const uint8_t* w2s_fused, uint8_t* w13,
                               uint8_t* w13s, uint8_t* w2, uint8_t* w2s, void* w13_bf16,
                               void* w2_bf16, int32_t* expert_map, hipStream_t stream);

/*
 * The layer with experts kept in bf16 (bx from mxfp4_moe_preshuffle_fused's
 * outputs; bx itself is host memory, read during the call).  Packed experts
 * run as in mxfp4_moe_forward; an excluded expert's rows are computed from its
 * bf16 weights on the bf16 x and the bf16 SwiGLU output in every activation
 * mode (no A4/A8 quantisation for them).  Workspace as mxfp4_moe_forward.  The
 * intermediates act, actq, acts, xq, xs and out32 are copied out as by
 * mxfp4_moe_forward_debug when non-NULL (all may be NULL).  Errors as
 * mxfp4_moe_forward, plus: bx NULL or, with n > 0, a NULL map or weight ->
 * NULL_POINTER; n < 0 or n > E_w -> BAD_ARGUMENT.
 */
int mxfp4_moe_forward_mixed(const mxfp4_moe_dims* d, const mxfp4_moe_bf16_experts* bx,
                            const void* x, const float* router_logits, const uint8_t* w13,
                            const uint8_t* w13s, const uint8_t* w2, const uint8_t* w2s,
                            int32_t top_k, float clamp_limit, void* out, void* workspace,
                            size_t workspace_bytes, void* act, uint8_t* actq, uint8_t* acts,
                            uint8_t* xq, uint8_t* xs, float* out32, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MXFP4_MOE_H */
