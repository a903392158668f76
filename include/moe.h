/*
 * moe.h -- C ABI of the MI355X (gfx950) BF16 Mixture-of-Experts expert path.
 *
 * One layer of the path is: router logits -> softmax top-k routing with
 * expert grouping -> grouped gate-up GEMM with SiLU-mul -> grouped
 * down-projection carrying the routing weight -> weighted top-k combine with
 * a sigmoid-gated shared-expert term.
 *
 * Sources (web pages, cited by title and section):
 *   [Issue 3094] vllm.cpp issue #3094, row "BACKEND-ROCM-BF16-MOE", row
 *       statement: ROCm lacks the BF16 grouped expert GEMMs (plain and
 *       gate-up + SiLU); numeric contract N1 (GEMM result narrowed to bf16
 *       before the activation), N2 (routing weight applied before the
 *       down-projection result is stored), N3 (the reduction must not apply
 *       the routing weights a second time).
 *   [PR 509] vllm.cpp PR #509 "feat(rocm): MoE combine/gate ops --
 *       SharedExpertGate, MoeCombine, MoeCombineGate": What changed (combine
 *       formulas), Honest gaps (ungrouped softmax router), review comment
 *       (f32/bf16 arms only, f16 refused with a named message; expert_out is
 *       the pair-major [T,K,H] bf16 buffer), rework commit (bit-exact combine:
 *       thread per element, sequential k, one store rounding, no
 *       contraction), routed_scale commit (one multiply on the finished routed
 *       sum before the shared add).
 *   [PR 523] keep-quant grouped expert GEMM, What changed / Honest gaps:
 *       grouping over expert ids; capture-safe scratch that never
 *       reallocates during reuse.
 *
 * Conventions common to every call
 *   - All data pointers are DEVICE pointers (hipMalloc'd or equivalent) of the
 *     current HIP device, owned by the caller. The library never allocates or
 *     frees, never synchronises, and keeps no state beyond a thread-local
 *     error string and a per-device "checked" flag.
 *   - bf16 tensors are passed as uint16_t bit patterns (IEEE bfloat16).
 *   - All tensors are dense row-major with the shapes given; base pointers of
 *     bf16/f32 tensors read or written with 16-byte vectors must be 16-byte
 *     aligned (stated per argument).
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *     enqueues work on it and returns; it is legal inside hipGraph capture
 *     once moe_init() has run outside capture.
 *   - Validation happens on the host before any launch. On failure the call
 *     returns a non-zero moe_status, launches nothing, leaves the outputs
 *     untouched and records a message naming the call, the argument and the
 *     missing piece (moe_last_error). A launch error maps to MOE_E_HIP.
 *     Device faults surface at the caller's next synchronisation.
 *   - A call with zero tokens (T == 0 or P == 0) returns MOE_OK and does
 *     nothing.
 *   - Limits: 1 <= K <= E, E <= 1024, K <= 32, H and I multiples of 8,
 *     T*K, T*E, T*K*I and T*K*H below 2^31 elements; the GEMM operands x and
 *     act below 2^30 elements, one expert's packed weights below 2^31 bytes.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_E_INVALID = 1,   /* null/misaligned pointer, non-finite scalar, bad flag */
  MOE_E_DTYPE = 2,     /* dtype arm not implemented (f16) or unknown        */
  MOE_E_SHAPE = 3,     /* a dimension outside the limits above              */
  MOE_E_WORKSPACE = 4, /* workspace smaller than the query returned          */
  MOE_E_HIP = 5        /* a HIP runtime error (wrong device arch, launch)    */
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_F16 = 2          /* exists only so that it can be refused by name */
} moe_dtype;

/* hipStream_t, passed as an opaque pointer so this header needs no HIP headers. */
typedef void* moe_stream_t;

/* Message of the last failed call on this thread ("" if none). Never NULL. */
const char* moe_last_error(void);

/* Checks that the current device is gfx950 and loads the code objects. Call
 * once per device before any hipGraph capture; the other calls do it on
 * first use. Returns MOE_E_HIP (with a message) on another architecture. */
moe_status moe_init(void);

/* Measurement only. Arms kernel timing for the next GEMM call
 * (moe_router_logits, moe_grouped_gemm_gateup_silu, moe_grouped_gemm_down,
 * moe_grouped_qgemm_gateup_silu, moe_grouped_qgemm_down), combine call
 * (moe_combine_gate) or probe call (moe_probe_hbm_read, moe_probe_mfma_bf16)
 * made by this host thread: its kernel is launched so that it records its
 * own start and end into `start` and `stop` (hipEvent_t created by the
 * caller), and hipEventElapsedTime(start, stop) then gives the kernel's
 * duration without the launch gap. The next such call disarms it whether or
 * not it launches (T = 0, a refused argument). Both NULL disarms; one NULL
 * is MOE_E_INVALID. Not for use under hipGraph capture. */
moe_status moe_time_next_gemm(void* start, void* stop);

/* Measurement only: the two ceilings the bench reads its figures against on
 * the chip at hand, beside the datasheet peaks. Each launches 262,144
 * threads (4,096 wavefronts) and writes one 32-bit value per thread to
 * `out` (device memory of at least moe_probe_out_values() values; caller
 * owned). A call armed by moe_time_next_gemm records its kernel's start and
 * end like a GEMM call. Errors: NULL or misaligned pointers and sizes out of
 * range give MOE_E_INVALID; launch failures MOE_E_HIP. */
size_t moe_probe_out_values(void);

/* Streaming read of `bytes` (a multiple of 16, at least 16) of the device
 * buffer `buf` (16-byte aligned), 16-byte loads; out[i] (uint32) = XOR of
 * every dword thread i read, so the XOR of all outputs is the XOR of every
 * dword of the buffer. */
moe_status moe_probe_hbm_read(const void* buf, size_t bytes, uint32_t* out, moe_stream_t stream);

/* Register-only loop of v_mfma_f32_32x32x16_bf16: every wavefront runs `iters`
 * (1 .. 2^20) iterations of 4 independent MFMAs (32,768 flops each) on bf16
 * operands read from `ops` (n_ops 8-value operands = 16 * n_ops bytes,
 * 16-byte aligned, 1 <= n_ops <= 2^26), i.e. moe_probe_mfma_flops(iters)
 * flops per launch; out[i] (f32) = sum of thread i's accumulators. */
moe_status moe_probe_mfma_bf16(const uint16_t* ops, size_t n_ops, int iters, float* out,
                               moe_stream_t stream);
double moe_probe_mfma_flops(int iters);

typedef enum {
  MOE_PACK_PLAIN = 0,  /* a matrix [R, K] (down projection: R = H, K = I) */
  MOE_PACK_GATEUP = 1  /* a gate-up matrix [2I, K]: gate rows [0, I), up rows [I, 2I) */
} moe_pack_kind;

/*
 * Packed expert weights: the weight format the grouped GEMMs read. Each
 * expert's matrix is cut into 1 KiB blocks of 16 rows x 32 k; inside a block
 * the 16-byte chunk q = 16*c + r holds W[16*rb + r][32*kb + 8*c .. +8], the
 * lane order of one 16x32 MFMA operand, so every weight load of a wavefront
 * is one contiguous 1 KiB. Rows past R and k past K are zero.
 *   MOE_PACK_PLAIN:  block (rb, kb) at byte (rb * nkb + kb) * 1024
 *   MOE_PACK_GATEUP: the gate block of output columns [16*cb, +16) and the
 *                    matching up block (rows I + [16*cb, +16)) side by side:
 *                    (cb, kb, f) at ((cb * nkb + kb) * 2 + f) * 1024, f = 0
 *                    gate, 1 up
 * with nkb = ceil(K / 32); experts follow one another. Packing is a layout
 * change done once when weights are loaded, not a step of the layer (the
 * pages' operands are the row-major W_gu [E,2I,H] and W_d [E,H,I]; the
 * arithmetic of the GEMMs is unchanged).
 * moe_packed_weight_bytes returns the size of the packed tensor (0 for
 * invalid arguments: E, R, K < 1, K not a multiple of 8, R odd for GATEUP).
 * moe_pack_weights converts w (bf16 [E, R, K], 16-byte aligned, device) into
 * packed (device, 16-byte aligned, moe_packed_weight_bytes bytes), stream-
 * ordered like every call, and fills the host descriptor *desc (not NULL)
 * that the grouped GEMMs take in place of a bare weight pointer. Limits:
 * E <= 1024, R * K below 2^30 elements. On any refusal *desc is left as it
 * was.
 */
size_t moe_packed_weight_bytes(int E, int R, int K, moe_pack_kind kind);

/* The layout tag of a descriptor filled by moe_pack_weights. */
#define MOE_WEIGHTS_PACKED_V1 0x4D4F4531u

/*
 * Host-side descriptor of a packed expert weight set: the weight argument of
 * moe_grouped_gemm_gateup_silu, moe_grouped_gemm_down and
 * moe_fused_expert_ffn. The row-major W_gu [E,2I,H] / W_d [E,H,I] of the
 * pages cannot be read by these kernels, and a bare device pointer cannot
 * say which layout it holds; so the calls take this descriptor, which only
 * moe_pack_weights (and moe_weights_slice) fill, and refuse with
 * MOE_E_INVALID and a message naming the argument any descriptor whose
 * layout tag is not MOE_WEIGHTS_PACKED_V1, whose kind is not the call's
 * (GATEUP for w_gu, PLAIN for w_d) or whose dimensions differ from the
 * call's (E, 2I x H for w_gu, H x I for w_d). The caller owns the struct
 * (plain host memory, read during the call only) and the device memory
 * `data` points at.
 */
typedef struct {
  uint32_t layout;       /* MOE_WEIGHTS_PACKED_V1 */
  int32_t kind;          /* moe_pack_kind */
  int32_t E, R, K;       /* experts, rows and reduced length of each expert's matrix */
  int32_t reserved;
  const void* data;      /* device: the packed blocks of expert 0 */
  uint64_t expert_bytes; /* bytes of one expert's packed matrix */
} moe_weights;

moe_status moe_pack_weights(const uint16_t* w, int E, int R, int K, moe_pack_kind kind,
                            uint16_t* packed, moe_weights* desc, moe_stream_t stream);

/* Experts [e0, e1) of a packed weight set as a descriptor of their own,
 * viewing the same device memory (each expert's packed matrix is
 * contiguous): the block of experts one rank owns when experts are split
 * across GPUs. Host only, no launch. MOE_E_INVALID for a descriptor not
 * filled by moe_pack_weights, MOE_E_SHAPE unless 0 <= e0 < e1 <= w->E. */
moe_status moe_weights_slice(const moe_weights* w, int e0, int e1, moe_weights* out);

/*
 * Router / gate logits helper (not a contract step; the router itself is the
 * ungrouped softmax top-k of [PR 509] Honest gaps).
 *   out[t,n] = f32( sum_h x[t,h] * w[n,h] )  (+ bias[n] as one f32 add)
 *   x    bf16 [T,H], 16-byte aligned          w    bf16 [N,H], 16-byte aligned
 *   bias f32 [N] or NULL                      out  f32 [T,N]
 * The sum is an f32 MFMA accumulation in the kernel's own order. N >= 1
 * (N = E for the router, N = 1 for the shared-expert gate logit).
 */
moe_status moe_router_logits(const uint16_t* x, int T, int H, const uint16_t* w, int N,
                             const float* bias, float* out, moe_stream_t stream);

/* Bytes of device workspace moe_route needs for (T, E, K): 0 up to 4096
 * routed pairs (T*K), else 4 bytes per (1024-pair segment, expert). The
 * workspace is scratch owned by the caller, 4-byte aligned, and may be
 * reused across calls on one stream; its contents on entry do not matter. */
size_t moe_route_workspace_bytes(int T, int E, int K);

/*
 * Softmax top-k routing with renormalisation and stable expert grouping
 * ([PR 509] Honest gaps: ungrouped softmax; [PR 523]: grouping by expert id).
 *   logits         f32 [T,E] (read only)
 *   topk_ids       int32 [T,K]: the K largest logits per token, descending,
 *                  ties to the lower expert id, NaN ranked as -inf
 *   topk_w         f32 [T,K]: w_k = e_k / (((e_0 + e_1) + ...) + e_{K-1}),
 *                  e_k = exp(l_k - l_0) with the library's bit-reproducible
 *                  f32 exp (Cody-Waite reduction + degree-7 Taylor)
 *   expert_offsets int32 [E+1]: offsets[e] = number of pairs routed to
 *                  experts below e; offsets[E] = T*K
 *   sorted_pairs   int32 [T*K]: pair indices p = t*K + k grouped by expert,
 *                  increasing p within an expert
 *   ws, ws_bytes   workspace of at least moe_route_workspace_bytes(T,E,K)
 *                  bytes (MOE_E_WORKSPACE if smaller; NULL allowed when 0)
 * Results are bit-identical run to run (no atomics decide an order).
 */
moe_status moe_route(const float* logits, int T, int E, int K, int32_t* topk_ids,
                     float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                     void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * For callers that cannot allocate (code under hipGraph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_route with the
 * grouping scratch held by the library instead of a caller workspace. Same
 * arguments (without ws, ws_bytes), results and errors as moe_route. The
 * library holds 1 MiB of scratch per GPU in a static device array (kept
 * until the process ends); T*K pairs over E experts need
 * moe_route_workspace_bytes(T, E, K) bytes of it (4 per (1024-pair segment,
 * expert)), so with E = 128 up to 2,097,152 pairs fit; larger sizes are
 * refused with MOE_E_WORKSPACE. Nothing in the scratch needs to start at
 * zero. It calls no allocator. Every call on one GPU shares that GPU's
 * scratch: calls that overlap on one GPU (on different streams, or from
 * different host threads) race and must be ordered by the caller. The
 * scratch's device address is looked up by moe_init (or by the first call on
 * a device): call moe_init on each device before capturing this call.
 */
moe_status moe_route_noalloc(const float* logits, int T, int E, int K, int32_t* topk_ids,
                             float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                             moe_stream_t stream);

typedef enum {
  MOE_SCORE_SOFTMAX = 0, /* softmax over all E experts */
  MOE_SCORE_SIGMOID = 1  /* sigmoid of each logit */
} moe_score;

typedef enum {
  MOE_GROUP_MAX = 0,     /* a group is scored by its largest selection value */
  MOE_GROUP_TOP2_SUM = 1 /* ... by the sum of its two largest */
} moe_group_score;

/*
 * General router: sigmoid or full-softmax scores, a selection bias and
 * group-limited selection, then the same grouping as moe_route. These are the
 * router forms [Issue 3094] (row statement: the DeepSeek-V2 / Dots3 grouped
 * and sigmoid router gaps) and [PR 509] (Honest gaps: grouped / bias /
 * noaux_tc forms) name as the gaps left; the arithmetic is read from the
 * DeepSeek-V2 and DeepSeek-V3 technical reports. Per token, f32, each
 * operation rounded on its own:
 *   s_e = sigmoid(l_e)                                  (MOE_SCORE_SIGMOID)
 *   s_e = z_e / S, z_e = exp(l_e - max_j l_j), S = sum of z in the order of a
 *         64-lane butterfly (lane e%64 adds its z in increasing e, then lanes
 *         l and l^m are added for m = 32, 16, 8, 4, 2, 1)  (MOE_SCORE_SOFTMAX)
 *   c_e = s_e + selection_bias[e] (selection_bias NULL: c_e = s_e); NaN
 *         ranks as -inf
 *   n_group > 1: experts form n_group groups of E/n_group consecutive ids; a
 *         group scores max c (MOE_GROUP_MAX) or the f32 sum of its two largest
 *         c (MOE_GROUP_TOP2_SUM); the topk_group best groups (ties to the
 *         lower group) stay allowed
 *   topk_ids: K rounds of the largest allowed c, ties to the lower id
 *   topk_w:   w_k = s of expert k (the bias steers selection only); with
 *             renormalize = 1, w_k / (((w_0 + w_1) + ...) + w_{K-1})
 * exp is the library's f32 exp (as in moe_route), the divides correctly
 * rounded. Limits: 1 <= n_group <= 64, n_group divides E, 1 <= topk_group <=
 * n_group, topk_group * E/n_group >= K (MOE_E_SHAPE otherwise);
 * renormalize in {0, 1}. selection_bias is f32 [E] device memory or NULL.
 * Outputs, workspace and the rest of the contract as moe_route.
 */
moe_status moe_route_scored(const float* logits, int T, int E, int K, moe_score score,
                            const float* selection_bias, int n_group, int topk_group,
                            moe_group_score group_score, int renormalize, int32_t* topk_ids,
                            float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                            void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Grouped gate-up GEMM with SiLU-mul ([Issue 3094] row statement, N1).
 * For sorted row q of expert e (p = sorted_pairs[q], token t = p / K):
 *   gu[j]    = bf16( f32( x[t] . w_gu[e,j] ) )          j < 2I   (N1)
 *   act[q,i] = bf16( silu(gu[i]) * gu[I+i] ),  silu(g) = g / (1 + exp(-g))
 *   x      bf16 [T,H], 16-byte aligned
 *   w_gu   descriptor of the gate-up weights W_gu [E,2I,H] (gate rows
 *          [0,I), up rows [I,2I)) packed by moe_pack_weights(..., E, 2I, H,
 *          MOE_PACK_GATEUP, ...); anything else is refused (see moe_weights)
 *   sorted_pairs, expert_offsets  as produced by moe_route(T, E, K); both
 *          NULL means identity rows (E must be 1 and K 1: a dense expert,
 *          e.g. the shared expert)
 *   act    bf16 [T*K, I] in sorted order, 16-byte aligned
 * Experts with no rows cost nothing. f32 accumulation on MFMA.
 */
moe_status moe_grouped_gemm_gateup_silu(const uint16_t* x, int T, int H,
                                        const moe_weights* w_gu, int E, int I, const int32_t* sorted_pairs,
                                        const int32_t* expert_offsets, int K, uint16_t* act,
                                        moe_stream_t stream);

/*
 * Grouped down-projection with the routing weight in the epilogue
 * ([Issue 3094] row statement, N2 and N3).
 *   y = f32( act[q] . w_d[e,h] );  expert_out[p,h] = bf16( y * pair_w[p] )
 *   stored at pair row p = sorted_pairs[q], so expert_out is [T,K,H].
 *   act    bf16 [P,I] in sorted order, 16-byte aligned
 *   w_d    descriptor of the down weights W_d [E,H,I] packed by
 *          moe_pack_weights(..., E, H, I, MOE_PACK_PLAIN, ...); anything
 *          else is refused (see moe_weights)
 *   sorted_pairs, expert_offsets  from moe_route, or both NULL (identity, E=1)
 *   pair_w f32 [P] (= topk_w viewed flat) or NULL for no multiply
 *   expert_out bf16 [P,H], 16-byte aligned
 */
moe_status moe_grouped_gemm_down(const uint16_t* act, int P, int I, const moe_weights* w_d,
                                 int E, int H, const int32_t* sorted_pairs,
                                 const int32_t* expert_offsets, const float* pair_w,
                                 uint16_t* expert_out, moe_stream_t stream);

/*
 * Weighted top-k combine with routed scale and an optional (gated) shared
 * term ([PR 509] What changed, rework and routed_scale commits). Per (t,h),
 * f32, each operation rounded on its own (no contraction):
 *   acc = +0; for k = 0..K-1: v = expert_out[t,k,h]; if (topk_w) v = topk_w[t,k]*v;
 *             acc = acc + v
 *   acc = acc * routed_scale
 *   if (shared): s = shared[t,h]; if (gate_logit) s = f32(bf16(sigmoid(gate_logit[t]) * s));
 *                acc = acc + s
 *   out[t,h] = bf16(acc) or acc (by out_dt)
 *   expert_out eo_dt [T,K,H]; topk_w f32 [T,K] or NULL (weights already applied);
 *   shared sh_dt [T,H] or NULL; gate_logit f32 [T] or NULL (ungated shared add);
 *   out out_dt [T,H]. eo_dt, sh_dt, out_dt in {MOE_F32, MOE_BF16}; MOE_F16 is
 *   refused with MOE_E_DTYPE. Tensor base pointers 16-byte aligned.
 *   routed_scale must be finite (1.0 is the neutral value).
 */
moe_status moe_combine_gate(const void* expert_out, moe_dtype eo_dt, int T, int K, int H,
                            const float* topk_w, float routed_scale, const void* shared,
                            moe_dtype sh_dt, const float* gate_logit, void* out,
                            moe_dtype out_dt, moe_stream_t stream);

/* Workspace bytes of moe_fused_expert_ffn: int32 counters for T tokens, E
 * experts, top-K, grouped (sorted_pairs set) or not; 0 for T <= 0. */
size_t moe_fused_expert_ffn_workspace_bytes(int T, int E, int K, int grouped);

/* Decode expert FFN in one launch (gate-up -> SiLU -> down, [Issue 3094] N1,
 * N2, N3): the same results as moe_grouped_gemm_gateup_silu followed by
 * moe_grouped_gemm_down on the same arguments (act written as by the first,
 * expert_out as by the second; the down k order may differ, so expert_out
 * agrees to the GEMM tolerance, not bit for bit), with no launch boundary
 * between the two: a row tile's down projection starts as soon as the act
 * rows of that tile are complete, while other tiles' gate-up work is still
 * running. Arguments as those two calls (w_gu and w_d descriptors of packed
 * weights, refused as there unless filled by moe_pack_weights, act [T*K, I]
 * and expert_out [T*K, H] bf16, pair_w may be NULL). Meant for decode (a few
 * rows per expert); it streams every tile, so with hundreds of rows per
 * expert the two calls are faster. On MI355X at 32 tokens x 128 experts
 * (H 2048, I 768) it takes about 185 us against 104 + 53 us for the two
 * calls (its down phase has to take the gate-up's 512-thread workgroup
 * shape, where alone it runs best at 192 threads): it is kept for callers
 * that want one launch, not for speed.
 * ws: moe_fused_expert_ffn_workspace_bytes(T, E, K, sorted_pairs != NULL)
 * bytes, 4-byte aligned, owned by the caller, zero-filled before its first
 * use. Every launch leaves the counters zero again, so the same ws serves the
 * next call on the same stream (calls that overlap on one ws race). Its last
 * int32 is a status word: nonzero after a launch means one of the kernel's
 * bounded waits gave up (it cannot happen when the hardware dispatches
 * workgroups in order); expert_out is then invalid, the counters are in
 * doubt, and the whole ws must be zero-filled again before the next call.
 * MOE_E_WORKSPACE for a short, NULL or misaligned ws. */
moe_status moe_fused_expert_ffn(const uint16_t* x, int T, int H, const moe_weights* w_gu,
                                const moe_weights* w_d, int E, int I, const int32_t* sorted_pairs,
                                const int32_t* expert_offsets, int K, const float* pair_w,
                                uint16_t* act, uint16_t* expert_out, void* ws, size_t ws_bytes,
                                moe_stream_t stream);

/*
 * Keep-quant grouped expert GEMMs ([PR 523] What changed: expert weights stay
 * in their GGUF block formats Q8_0 / Q4_K / Q5_K / Q6_K, activations are
 * quantized on the fly by the Q8_0 and Q8_K quantizers, dot products run per
 * block with an integer core). Weight types, by GGUF type number:
 *   MOE_Q8_0: per 32 weights, 34 bytes = f16 d, 32 int8 quants (w = d q)
 *   MOE_Q4_K: per 256, 144 bytes = f16 d, f16 dmin, 12 bytes of six-bit
 *             sub-block scales and mins, 128 bytes of 4-bit quants
 *   MOE_Q5_K: per 256, 176 bytes = as Q4_K with 32 bytes of fifth bits
 *             between the scales and the 4-bit quants
 *   MOE_Q6_K: per 256, 210 bytes = 128 bytes of low nibbles, 64 bytes of
 *             2-bit high parts, 16 int8 scales of 16-value sub-blocks, f16 d
 * A weight matrix [R, K] is R rows of K/(values per block) blocks, experts
 * one after another; the base pointer is 16-byte aligned. K-quant weights
 * pair with Q8_K activations, Q8_0 weights with Q8_0 activations. Per
 * (super-)block the dot product of a weight row and an activation row is
 *   Q4_K, Q5_K: d_w d_x sum_j sc_j (sum_{l in j} q_l q8_l) - dmin_w d_x sum_j m_j bsum_j
 *   Q6_K:       d_w d_x sum_j sc_j (sum_{l in j} q6_l q8_l)
 *   Q8_0:       d_w d_x sum_l q_l q8_l
 * (integer inside, one f32 step per super-block or block, f32 sum over the
 * row). The reduced dimension (H for gate-up, I for down) must be a positive
 * multiple of 256 for every weight type, and one expert's blocks must stay
 * below 2^31 bytes.
 */
typedef enum { MOE_Q8_0 = 8, MOE_Q4_K = 12, MOE_Q5_K = 13, MOE_Q6_K = 14 } moe_qtype;

/* Bytes of the Q8_K buffer of R rows of K values (K a positive multiple of
 * 256; 0 otherwise or for R = 0). Layout, each section 256-byte aligned:
 * int8 quants [R, K], then f32 scales [R, K/256], then int32 sums of 16
 * quants [R, K/16]. */
size_t moe_q8k_bytes(int R, int K);

/* Q8_K quantization of bf16 rows x [R, K] (16-byte aligned) into xq
 * (moe_q8k_bytes(R, K) bytes, 16-byte aligned): per 256 values, the first
 * entry of largest magnitude gives iscale = -127 / max, q = min(127,
 * round-half-even(iscale * x)), d = 1 / iscale (f32); an all-zero block gives
 * d = 0, q = 0. Activations must be finite. */
moe_status moe_quantize_q8k(const uint16_t* x, int R, int K, void* xq, moe_stream_t stream);

/* Bytes of the Q8_0 buffer of R rows of K values (K a positive multiple of
 * 32; 0 otherwise or for R = 0). Layout, each section 256-byte aligned: int8
 * quants [R, K], then f16 scales [R, K/32]. */
size_t moe_q8_0_bytes(int R, int K);

/* Q8_0 quantization of bf16 rows x [R, K] (16-byte aligned) into xq
 * (moe_q8_0_bytes(R, K) bytes, 16-byte aligned), per 32 values: amax = max
 * |x|, d = amax / 127, id = 1 / d (0 when d = 0), q = round-half-away-from-
 * zero(x * id) (f32 arithmetic), d stored as f16 (round to nearest even).
 * Activations must be finite. */
moe_status moe_quantize_q8_0(const uint16_t* x, int R, int K, void* xq, moe_stream_t stream);

/* Keep-quant grouped gate-up with SiLU-mul ([PR 523]; [Issue 3094] N1):
 *   g, u = keep-quant dots of the quantized row of token t = sorted_pairs[q]
 *          / K with gate row c and up row I + c of expert e (w_gu [E, 2I, H]
 *          in format wt)
 *   act[q, c] = bf16(silu(bf16(g)) * bf16(u))
 * xq: moe_quantize_q8k of x [T, H] for the K-quants, moe_quantize_q8_0 for
 * MOE_Q8_0; routing arguments, act and errors as
 * moe_grouped_gemm_gateup_silu (NULL routing = one dense expert, E = K = 1);
 * an unknown wt gives MOE_E_DTYPE. */
moe_status moe_grouped_qgemm_gateup_silu(const void* xq, int T, int H, const void* w_gu,
                                         moe_qtype wt, int E, int I, const int32_t* sorted_pairs,
                                         const int32_t* expert_offsets, int K, uint16_t* act,
                                         moe_stream_t stream);

/* Keep-quant grouped down projection ([PR 523]; [Issue 3094] N2, N3):
 *   y = keep-quant dot of the quantized row q of act with row h of expert
 *       e's w_d [E, H, I] (format wt);  expert_out[p, h] = bf16(y *
 *       pair_w[p]), p = sorted_pairs[q]
 * actq: the quantizer output paired with wt, of act [P, I]; the rest as
 * moe_grouped_gemm_down. */
moe_status moe_grouped_qgemm_down(const void* actq, int P, int I, const void* w_d, moe_qtype wt,
                                  int E, int H, const int32_t* sorted_pairs,
                                  const int32_t* expert_offsets, const float* pair_w,
                                  uint16_t* expert_out, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
