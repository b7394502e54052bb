/* moe.h -- C ABI of the routed mixture-of-experts layer for MI355X (gfx950).
 *
 * One MoE layer of the model the Strata pages describe: per token a router
 * GEMV over 512 experts, the 10 highest-scoring experts with softmax gate
 * weights, a lookup of each chosen expert in a resident-expert slot table
 * (hits are computed, misses are listed), a dequant-fused low-bit SwiGLU
 * expert FFN and a gate-weighted combine with an always-on shared expert.
 * Sources (page titles and sections):
 *   [MD] ModelDock, "Strata はなぜ少ない VRAM でも速いのか" (why Strata is fast
 *        with little VRAM): section "問題" (48 layers x 512 experts, 10 chosen
 *        per token; the shared expert is among the weights every token uses),
 *        section "1 トークン、三者の分担" (router on the GPU, chosen ids looked
 *        up, resident experts run on the GPU, the GPU sums the results),
 *        section "粗から細へ" and its placement figure (slot table of
 *        individual resident experts, 57-109 per layer), section
 *        "予測してから検証する" (a verify step of 1 + up to 3 draft tokens
 *        reads each expert once), section "長いプロンプトを読む" (prefill:
 *        thousands of tokens hit nearly every expert).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers owned by the caller unless stated; the
 *    library keeps none of them after the call returns.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronise the host.  They never allocate device
 *    memory: scratch space is the caller's workspace `ws` of `ws_bytes`
 *    bytes, at least moe_workspace_size() and 256-byte aligned.
 *  - Arguments are validated on the host before any launch.  On any error
 *    nothing is launched, nothing is written and a non-zero moe_status is
 *    returned.  A device fault surfaces at the caller's next synchronisation.
 *    T = 0 is a valid no-op (MOE_OK).  NaN/Inf inputs give unspecified
 *    values (never out-of-bounds accesses).
 *  - Row-major layouts; "K" is the contiguous (input) dimension.
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
  MOE_ERR_INVALID = 1,      /* bad shape, null pointer, misalignment, k > E ... */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not implemented (format, T too large) */
  MOE_ERR_WORKSPACE = 3,    /* ws_bytes smaller than moe_workspace_size() */
  MOE_ERR_DEVICE = 4        /* a HIP call failed, or a fused launch gave up (moe_layer_check) */
} moe_status;

/* Weight formats.  Q2B32 / Q4B32: blocks of 32 consecutive weights along K
 * of each row, one fp16 scale d and one fp16 min m per block, weight =
 * d * q + m with q the unsigned 2- or 4-bit code.  The code of column c of a
 * row sits bits*(c mod (8/bits)) bits up in byte c*bits/8 of that row (low
 * bits first).  This is the "scale + min" low-bit block family of the
 * quantised expert files the pages name (Q2_0 and friends); the exact 32-
 * weight affine block is this library's definition. */
typedef enum {
  MOE_W_F32 = 0,   /* fp32, [rows][cols] */
  MOE_W_BF16 = 1,  /* bf16 bits, [rows][cols] (router only) */
  MOE_W_Q2B32 = 2, /* 2-bit codes, 3.0 bits per weight with scale and min */
  MOE_W_Q4B32 = 3  /* 4-bit codes, 5.0 bits per weight with scale and min */
} moe_wfmt;

/* One matrix pool: `n` matrices of [rows][cols] stacked by slot.
 *  F32:   data = float  [n][rows][cols]; scale = min = NULL.
 *  Q2/Q4: data = codes  [n][rows*cols*bits/8] bytes (16-byte aligned);
 *         scale, min = fp16 bits [n][rows][cols/32] (4-byte aligned). */
typedef struct {
  int32_t fmt;
  const void* data;
  const uint16_t* scale;
  const uint16_t* min;
} moe_mat;

/* One layer.  Expert pools are indexed by SLOT: gate and up [S][I][H], down
 * [S][H][I], all in one expert format (F32, Q2B32 or Q4B32).
 * slot_of_expert[E] maps an expert id to its slot or -1 (not resident); NULL
 * means every expert is resident at slot = id (then num_slots must be E).
 * Several layers may share one pool (a global slot table).  The shared expert
 * (sh_*) uses the same format and shapes with n = 1; sh_gate.data == NULL
 * means the layer has none.  Router weights [E][H] are F32 or BF16;
 * router_bias [E] fp32 may be NULL.  Limits: 1 <= k <= min(E, 32), E <= 1024,
 * H and I multiples of 32 (of 64 for Q2B32), H <= 8192, I <= 4096,
 * 1 <= num_slots <= 16384.
 * usage_counts [E] uint32 may be NULL; when set, moe_layer and
 * moe_resolve_slots add 1 to usage_counts[e] for every choice of expert e
 * (hits and misses, every token), with device-scope atomic adds: the counts
 * moe_slot_refresh ranks experts by. */
typedef struct {
  int32_t E, k, H, I, num_slots;
  int32_t router_fmt;
  const void* router_w;
  const float* router_bias;
  const int32_t* slot_of_expert;
  moe_mat gate, up, down;
  moe_mat sh_gate, sh_up, sh_down;
  uint32_t* usage_counts;
} moe_layer_desc;

/* One missed (not resident) expert of one token, with its gate weight. */
typedef struct {
  int32_t expert;
  int32_t token;
  float gate;
} moe_miss;

/* Largest T accepted by moe_layer (a decode step, a 1 + 3 draft verify batch
 * and the 16-token slot-table step all fit). */
#define MOE_LAYER_MAX_T 16

const char* moe_status_string(int32_t status);

/* Library version (major * 10000 + minor * 100 + patch). */
int32_t moe_version(void);

/* Workspace bytes needed by every call below for this layer shape and T. */
moe_status moe_workspace_size(const moe_layer_desc* desc, int32_t T, size_t* bytes);

/* Router and gates ([MD] "問題", "1 トークン、三者の分担").
 * x: bf16 bits [T][H].  logit[t][e] = sum_h x[t][h] W[e][h] + bias[e] in fp32
 * accumulation.  topk_idx [T][k] int32: the k largest logits per token in
 * descending order, the lower expert id first on equal logits (-0.0 equals
 * +0.0).  topk_gate [T][k] fp32: softmax over the k selected logits. */
moe_status moe_route(const moe_layer_desc* desc, const uint16_t* x, int32_t T,
                     int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes,
                     void* stream);

/* Slot resolution, miss list and buckets ([MD] "1 トークン、三者の分担",
 * placement figure of "粗から細へ").  Pair p = t*k + j.
 *  slot_idx [T][k]: slot of each chosen expert, -1 when not resident
 *    (topk_idx outside [0, E), or slot_of_expert outside [-1, S), count as
 *    not resident).
 *  miss [T*k] + miss_off [T+1]: the misses as (expert, token, gate) in
 *    (t, j) order; token t's are miss[miss_off[t] .. miss_off[t+1]).  The
 *    gate is copied bit for bit from topk_gate.
 *  bucket_off [S+1], bucket_pair [T*k]: hit pairs sorted stably by slot
 *    (i.e. by (slot, t, j)); slot s owns bucket_pair[bucket_off[s] ..
 *    bucket_off[s+1]).  Entries past bucket_off[S] are left untouched. */
moe_status moe_resolve_slots(const moe_layer_desc* desc, const int32_t* topk_idx,
                             const float* topk_gate, int32_t T, int32_t* slot_idx,
                             int32_t* bucket_off, int32_t* bucket_pair, moe_miss* miss,
                             int32_t* miss_off, void* ws, size_t ws_bytes, void* stream);

/* Expert FFN of every bucketed pair and of the shared expert ([MD]
 * "1 トークン、三者の分担", "長いプロンプトを読む").  For a pair p = t*k + j in
 * slot s's bucket: a = G_s x_t, u = U_s x_t, h = silu(a) * u, pair_out[p] =
 * D_s h (fp32 [T*k][H]; rows of pairs in no bucket are left untouched).
 * shared_out [T][H] fp32 = the same FFN with the shared expert (ignored and
 * may be NULL when the layer has none).  Each slot's weights are read once
 * for all of its tokens.  Small T runs dequant-fused GEMVs; large T (>= 256
 * tokens with Q2/Q4 experts) runs an fp16-MFMA grouped GEMM whose weights
 * are dequantised to fp16 tiles (fp32 accumulation). */
moe_status moe_expert_ffn(const moe_layer_desc* desc, const uint16_t* x, int32_t T,
                          const int32_t* bucket_off, const int32_t* bucket_pair,
                          float* pair_out, float* shared_out, void* ws, size_t ws_bytes,
                          void* stream);

/* The expert FFN with the combine fused into it ([MD] "長いプロンプトを読む":
 * prefill streams each expert over all of its tokens, and the GPU sums the
 * expert results).  y [T][H] fp32 is ACCUMULATED: for every pair p = t*k + j
 * in a slot's bucket, y[t] += topk_gate[p] * D_s h (h as for moe_expert_ffn),
 * and y[t] += the shared expert's output (weight 1) when the layer has one.
 * Pairs in no bucket (misses) add nothing.  With y zeroed first this is
 * moe_expert_ffn followed by moe_combine, without the [T*k][H] pair outputs
 * in memory.  The additions are device-scope float atomics, so y's
 * summation order (and its last bits) can differ from run to run.  Same
 * paths (GEMV or grouped GEMM), workspace and errors as moe_expert_ffn;
 * topk_gate [T][k] as moe_route writes it. */
moe_status moe_expert_ffn_accum(const moe_layer_desc* desc, const uint16_t* x, int32_t T,
                                const int32_t* bucket_off, const int32_t* bucket_pair,
                                const float* topk_gate, float* y, void* ws, size_t ws_bytes,
                                void* stream);

/* Combine ([MD] "1 トークン、三者の分担": the GPU sums the expert results).
 * y[t] = shared_out[t] + sum over j = 0..k-1 with slot_idx[t][j] >= 0 of
 * topk_gate[t][j] * pair_out[t*k+j], j ascending, fp32.  shared_out may be
 * NULL (no shared expert). */
moe_status moe_combine(const moe_layer_desc* desc, int32_t T, const int32_t* slot_idx,
                       const float* topk_gate, const float* pair_out, const float* shared_out,
                       float* y, void* stream);

/* The whole layer for decode and verify batches (1 <= T <= MOE_LAYER_MAX_T):
 * route, resolve, FFN of the hit experts (each read once), shared expert and
 * combine.  Outputs as above: y [T][H] fp32 (the misses are NOT in y: they
 * are listed in miss/miss_off for another tier), topk_idx, topk_gate
 * [T][k], slot_idx [T][k] (may be NULL), miss [T*k], miss_off [T+1].
 * When T*k <= 256 (and the router is BF16 for Q2/Q4 experts) this is one
 * persistent launch whose workgroups hand over through flags kept at the
 * start of ws, in a region no other call touches: the workspace must be
 * zero before its first moe_layer call (allocate it zeroed once); every call
 * leaves the flags ready for the next.  That launch sums the experts into y with
 * device-scope float atomics, so y can differ between runs in the last bits
 * (the gate-weighted terms are added in no fixed order).  A workspace serves one moe_layer call at a time,
 * and the launch sizes its grid to the workgroups the device holds at once,
 * so it should not share the GPU with a kernel that keeps some of them
 * from running: every wait of the launch is bounded (moe_set_wait_budget),
 * and a launch that runs out of it gives up instead of hanging -- see
 * moe_layer_check.  Other shapes run the separate steps in sequence. */
moe_status moe_layer(const moe_layer_desc* desc, const uint16_t* x, int32_t T, float* y,
                     int32_t* topk_idx, float* topk_gate, int32_t* slot_idx, moe_miss* miss,
                     int32_t* miss_off, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the static hand-off region moe_layer_noalloc uses on each GPU. */
#define MOE_LAYER_SCRATCH_BYTES (16u << 20)

/* moe_layer for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument.  The fused launch hands over through a static device
 * array of the library, MOE_LAYER_SCRATCH_BYTES on each GPU it runs on,
 * held until the process ends and cleared (by a kernel on `stream`) before
 * the first call on that GPU.  Every call on one GPU shares that GPU's
 * array, which carries the calls' sequence state from one call to the next:
 * calls that overlap on one GPU (several streams or host threads at once)
 * race and must not be made.  Only shapes that take the fused launch are
 * accepted (T * k <= 256, a BF16 router for Q2/Q4 experts, limits as for
 * moe_layer) and only while the hand-off region they need fits the array
 * (E <= 1024, k <= 32, I <= 4096 always do); others return
 * MOE_ERR_UNSUPPORTED and launch nothing.  Arguments, outputs and errors
 * as moe_layer; slot_idx may be NULL.  moe_layer_check(NULL, 0, stream)
 * reports whether a call on this GPU gave up a bounded wait, and clears the
 * array again if one did.  The call allocates nothing (no hipMalloc, no
 * allocating library routine). */
moe_status moe_layer_noalloc(const moe_layer_desc* desc, const uint16_t* x, int32_t T, float* y,
                             int32_t* topk_idx, float* topk_gate, int32_t* slot_idx,
                             moe_miss* miss, int32_t* miss_off, void* stream);

/* Whether the fused moe_layer calls made on workspace ws completed: MOE_OK,
 * or MOE_ERR_DEVICE when one of them gave up a bounded wait (for example
 * because another kernel kept some of its workgroups from running for
 * longer than the budget).  Such a call's outputs are unspecified (it never
 * accesses memory out of bounds), and every later moe_layer call on the
 * same workspace returns at once without writing anything, until the caller
 * zeroes the workspace again.  This call waits for the work queued on
 * `stream` and reads 4 bytes of ws: a host synchronisation, meant for
 * checks outside the hot path.  ws NULL checks the static region of
 * moe_layer_noalloc on the current GPU instead (and, when a call on it
 * gave up, clears it so that later calls work again).  ws not NULL and
 * ws_bytes < 256: MOE_ERR_INVALID. */
moe_status moe_layer_check(const void* ws, size_t ws_bytes, void* stream);

/* Budget of every wait of the fused moe_layer launch, in nanoseconds of the
 * GPU's real-time counter, counted from each workgroup's start (0 restores
 * the default of 100 ms).  hold != 0 is a test hook: workgroup 0 of every
 * later fused launch first waits on a word that nothing writes, so the
 * launch runs out of its budget, marks its workspace failed, and every
 * workgroup still exits normally.  Process-wide, read when a call is
 * issued. */
void moe_set_wait_budget(uint64_t ns, int32_t hold);

/* Diagnostics: phase stamps of later fused moe_layer launches.  trace is a
 * device buffer of 32 uint64 words per workgroup of the launch (one per
 * compute unit; 1024 rows always suffice), or NULL to stop.  Row b holds
 * workgroup b's real-time counter stamps (100 MHz) at: 0 start, 2 tokens
 * staged, 3 router/shared tasks of wave 0 done, 4 every logit seen by wave 0,
 * 11 by every wave, 5 routing done, 6 wave 0's gate/up done, 7 the last
 * wave's gate/up done, 12 down phase entered, 13 the first down unit's h
 * present, 8 first h staged, 9 down done, 10 end; word 1 is the XCD it ran
 * on, words 14 and 15 thread 0's poll rounds for that h and (one token)
 * for the logits; words 16-20 steps of routing (candidates listed, second
 * barrier (one token only), ranks, gates, resolution), word 21 the last
 * wave's router/shared tasks done, and 24-27 steps of the first down
 * unit's staging (two barriers, h converted, staging barrier).
 * Every launch overwrites the rows it writes.  Traced calls run a separate
 * instance of the fused kernel (the untraced one carries no stamps); calls
 * with fixed-order sums (moe_set_deterministic) are not traced.
 * Process-wide, read when a call is issued. */
void moe_set_trace(uint64_t* trace);

/* Order of the sums into y of later fused moe_layer launches (and of
 * moe_layer_noalloc).  on == 0 (the default): every down-projection unit
 * adds its gate-weighted rows into y with float atomics, whose order varies
 * from run to run, so y may differ in its last bits between identical calls
 * (the combine's definition, [MD] section "1 トークン、三者の分担", fixes
 * the value, not the order; [MD] "代償" accepts last-bit differences).
 * on != 0: the units publish their rows to the hand-off region instead, and
 * y[t][r] is summed over the hit choices in choice order j = 0 .. k-1, then
 * the shared expert, by one thread: y is bit-identical between identical
 * calls, whatever the grid size or timing.  Costs one more poll round trip
 * per launch.  Process-wide, read when a call is issued. */
void moe_set_deterministic(int32_t on);

/* ---- Adaptive slot table ([MD] section "粗から細へ" and its placement
 * figure: each card fills its expert slots by a usage ranking, and an
 * adaptive tier swaps at most 96 experts every 4 rounds toward the experts
 * the conversation actually uses, raising the share served from the card).
 *
 * One pool of num_slots expert slots serves L layers (a global slot table):
 * layer l's table is slot_of + l*E (its moe_layer_desc.slot_of_expert) and
 * its counts usage + l*E (its moe_layer_desc.usage_counts).  Expert j =
 * l*E + e.  All arrays are device memory; the store may also be host memory
 * the device can read (pinned, allocated as such by the caller). */
typedef struct {
  int32_t L, E, H, I, num_slots;
  moe_mat gate, up, down;              /* the pool: [num_slots] matrices each */
  moe_mat store_gate, store_up, store_down;  /* every expert: [L*E] matrices each, index j */
  uint32_t* usage;     /* [L*E] choice counts since the last refresh */
  int32_t* slot_of;    /* [L*E] slot of expert j, or -1 */
  int32_t* expert_of;  /* [num_slots] expert j held by the slot, or -1 (free) */
} moe_slot_pool;

/* Largest max_swaps of one refresh. */
#define MOE_REFRESH_MAX_SWAPS 1024

moe_status moe_slot_refresh_workspace_size(const moe_slot_pool* pool, size_t* bytes);

/* One refresh.  With u(j) = min(usage[j], 65535):
 *  candidates = experts j with slot_of[j] < 0 and u(j) > 0, ordered by u
 *    descending, then j ascending;
 *  victims = free slots (expert_of[s] < 0) by s ascending, then occupied
 *    slots by u(expert_of[s]) ascending, then s ascending;
 *  swap i pairs candidate i with victim i for i = 0, 1, ... while i <
 *    max_swaps, both lists last, and the victim is free or u(candidate) >
 *    u(victim's expert).
 * Each swap copies the candidate's gate/up/down planes from the store into
 * the victim slot, sets slot_of[old] = -1 (old = the victim's expert, if
 * any), slot_of[new] = s and expert_of[s] = new.  Then every count is
 * halved (usage[j] >>= 1), so recent rounds weigh most.  swaps [max_swaps]
 * [3] int32 receives (s, new, old or -1) for i < *n_swaps; n_swaps is one
 * device int32.  Stream-ordered: layer calls issued after it on the same
 * stream see the new tables and weights; calls in flight on other streams
 * must not use the pool meanwhile.  Limits: L*E <= 65536, num_slots <=
 * 16384, 0 <= max_swaps <= MOE_REFRESH_MAX_SWAPS; formats as for
 * moe_layer_desc (all six pools in one expert format). */
moe_status moe_slot_refresh(const moe_slot_pool* pool, int32_t max_swaps, int32_t* swaps,
                            int32_t* n_swaps, void* ws, size_t ws_bytes, void* stream);

/* Prefill layer in chunks ([MD] "長いプロンプトを読む": a long prompt is read
 * in chunks, up to 8,192 tokens by default and more when configured, and the
 * transfers of one step overlap the computation of another, each expert
 * serving a whole chunk).  Here the overlap is within the layer: the routing
 * of the next chunk runs beside the expert work of the current one.  The
 * prompt's T tokens
 * are cut into chunks of `chunk` tokens (the last one shorter; chunk >= T:
 * one chunk).  For each chunk: moe_route + moe_resolve_slots on aux_stream,
 * then moe_expert_ffn + moe_combine on stream, so chunk c + 1 is routed
 * while chunk c's experts run.  aux_stream NULL: everything on stream.  The
 * call orders itself after work already queued on stream, and on return
 * every launch is ordered before later work on stream.  Outputs: y [T][H]
 * fp32 (misses, if the slot table has any, contribute nothing, as in
 * moe_combine); topk_idx, topk_gate and slot_idx [T][k] of every token.  No
 * miss list (moe_resolve_slots gives one).  ws: moe_prefill_workspace_size
 * bytes (one full workspace plus the chunk's buckets, pair and shared
 * outputs, twice when there are several chunks), 256-byte aligned.  Events
 * are made once per device and host thread; calls on one device from
 * several host threads at once are not supported. */
moe_status moe_prefill_workspace_size(const moe_layer_desc* desc, int32_t T, int32_t chunk,
                                      size_t* bytes);
moe_status moe_prefill_layer(const moe_layer_desc* desc, const uint16_t* x, int32_t T,
                             int32_t chunk, float* y, int32_t* topk_idx, float* topk_gate,
                             int32_t* slot_idx, void* ws, size_t ws_bytes, void* stream,
                             void* aux_stream);

/* Acceptance of a verify pass ([MD] "予測してから検証する": a draft layer
 * proposes up to 3 next tokens, one pass of the model checks them all, keeps
 * the drafts the model agrees with and adds one token of its own, so the
 * output equals greedy decoding token for token).
 *  logits [T][V] fp32: row i is the model's prediction after input i of the
 *    verify batch (input 0 = the last accepted token, input i = draft i).
 *  draft [T-1] int32: the draft tokens (may be NULL when T = 1).
 * With g_i = the index of the largest logit of row i (the lowest index on
 * equal logits; -0.0 equals +0.0), drafts are kept while draft[i] == g_i;
 * with a kept, out_tokens[0 .. a] = g_0 .. g_a (the kept drafts, then the
 * model's own token) and *n_out = a + 1 (device int32).  out_tokens [T]:
 * entries past a receive g_i too.  Limits: 1 <= T <= 64, 1 <= V <= 2^26.
 * ws: moe_verify_workspace_size bytes, 256-byte aligned.  Async on stream. */
moe_status moe_verify_workspace_size(int32_t T, int32_t V, size_t* bytes);
moe_status moe_verify_accept(const float* logits, int32_t T, int32_t V, const int32_t* draft,
                             int32_t* out_tokens, int32_t* n_out, void* ws, size_t ws_bytes,
                             void* stream);

/* Host tier: the listed misses computed on the CPU ([MD] "1 トークン、三者の
 *分担": experts that are not on the card are computed by the CPU next to the
 * RAM that holds them, and the results are summed with the card's).
 * Unlike the calls above, every pointer here is a HOST pointer and the call
 * is synchronous; it uses no GPU.
 *  gate, up [n][I][H] and down [n][H][I]: the layer's experts indexed by
 *    expert id (n >= E), one format (F32, Q2B32 or Q4B32; layouts as for
 *    moe_mat, in host memory).
 *  x: bf16 bits [T][H], the layer input.  miss, miss_off: a miss list as
 *    moe_layer / moe_resolve_slots write it (host copies): token t's misses
 *    are miss[miss_off[t] .. miss_off[t+1]), each with token t, an expert in
 *    [0, E) named at most once per token, and its gate weight.
 *  y [T][H] fp32, accumulated: y[t] += gate * D_e(silu(G_e x_t) * U_e x_t)
 *    for every miss, in fp32.  With y holding moe_layer's output for a
 *    partial slot table, y becomes the layer's output with every expert
 *    resident (up to rounding).
 * Each missed expert's weights are read once for all of its tokens.  The
 * additions into each element of y happen in one fixed order (experts by
 * ascending id), so the result does not depend on n_threads (<= 0: the
 * hardware concurrency).  Invalid arguments or list: MOE_ERR_INVALID and y
 * untouched.  The dot products use AVX-512 when the CPU has it; the
 * environment variable MOE_HOST_ISA=generic, read at the first call,
 * selects plain C++ instead. */
moe_status moe_host_miss_ffn(int32_t E, int32_t H, int32_t I, moe_mat gate, moe_mat up,
                             moe_mat down, const uint16_t* x, int32_t T, const moe_miss* miss,
                             const int32_t* miss_off, float* y, int32_t n_threads);

/* Which code moe_host_miss_ffn runs: 1 = AVX-512, 0 = plain C++. */
int32_t moe_host_isa(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
