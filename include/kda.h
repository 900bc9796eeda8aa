/*
 * kda.h -- C ABI of libkda, the MI355X (gfx950) implementation of the Kimi
 * Delta Attention (KDA) layer's inference hot path: a fused single-launch
 * decode step (and its multi-token form for speculative verification), a
 * chunked varlen prefill that writes recurrent-state checkpoints, the
 * copy-on-write state copies used to resume from them, and the layer's input
 * and output projections.  The host-side prefix cache of states has its own
 * header, kda_prefix_cache.h.
 *
 * The layer, per sequence and head (dk key channels, dv value channels):
 *   a   = SiLU(causal depthwise conv of width 4 over the raw q | k | v channels)
 *   q^  = a_q / sqrt(|a_q|^2 + l2_eps),  k^ = a_k / sqrt(|a_k|^2 + l2_eps),  v^ = a_v
 *   S_t = (I - beta_t k^ k^T) Diag(exp g_t) S_{t-1} + beta_t k^ v^T     (dk x dv, fp32)
 *   o_t = S_t^T q^
 *   y_t = o_t / sqrt(mean(o_t^2) + rms_eps) * norm_w * sigmoid(z_t)
 * The pages this follows: vLLM blog "A Preview of Production-Scale Kimi K3
 * Support on vLLM" (sections "The Hardest Part: Prefix Caching for KDA" and
 * "KDA prefill and decode") and agentlenshq "vLLM Kimi K3 Support" (sections
 * "Hybrid KV-Cache Management", "Fused Kernels and Metadata Optimization" and
 * "Agentic Cache Retention Policies").  They describe the parts (recurrent
 * state plus short conv state per layer, a decode fusing conv, state update,
 * output gate and normalisation into one launch, a prefill that gathers the
 * initial states in one operation, checkpoints at fixed intervals and at
 * prompt ends, copy-on-write on a prefix hit); the equation above is the
 * gated delta rule with per-channel decay that they name.
 *
 * Conventions shared by every call
 * --------------------------------
 * Ownership: the caller owns every buffer.  The library allocates nothing,
 *   keeps no pointer after a call returns, and holds no global mutable state
 *   apart from a thread-local error message and, for
 *   kda_prefill_varlen_static, one static device buffer per device and its
 *   address.
 * Execution: every call enqueues its kernels on `stream` (a hipStream_t; NULL
 *   means the null stream) and returns without synchronising.  A fault inside
 *   a kernel surfaces at the caller's next synchronisation.
 * Errors: calls return a kda_status.  All argument checks run on the host
 *   before the first launch; on any error nothing is launched and
 *   kda_last_error() describes the problem.  Slot ids are device data and are
 *   checked inside the kernels: an out-of-range id is skipped (its outputs are
 *   filled with NaN where the call has outputs) instead of being dereferenced.
 * Pointers: device pointers must be 16-byte aligned unless a call states
 *   otherwise.
 * Layouts (row-major, innermost last; T = tokens of the call, S = slots):
 *   q, k      [T][H][dk]   activation dtype       v, z, out [T][H][dv]  activation dtype
 *   g         [T][H][dk]   fp32 (log decay, <= 0) beta      [T][H]      fp32
 *   conv_w    [H][2dk+dv][4] fp32 (per head: q channels, then k, then v;
 *             tap 3 multiplies the current token, tap 0 the token 3 back)
 *   norm_w    [dv] fp32, shared by all heads
 *   state     [S][H][dk][dv] state dtype (pool of recurrent states; also
 *                                       the checkpoint format)
 *   conv      [S][H][2dk+dv][3] activation dtype (raw inputs of the last 3
 *                                       tokens, index 0 = oldest)
 * Supported shapes: dk == dv in {32, 64, 128}; conv width 4; H >= 1.  One
 *   exception: kda_prefill_varlen with fp32 activations takes dk == dv in
 *   {32, 64} only (its LDS staging of 64 fp32 token rows at 128 does not fit
 *   a workgroup's 160 KB) and returns KDA_ERR_UNSUPPORTED for 128.
 * Gates: every call accepts any log-decay g <= 0, including -inf (that
 *   channel of the state is forgotten).  A NaN gate gives NaN results.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,  /* NULL / misaligned pointer, bad size or count */
    KDA_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement */
    KDA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
    KDA_ERR_HIP = 4           /* the HIP runtime refused a launch */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Flags of kda_prefill_varlen (bitwise or). */
typedef enum {
    KDA_PREFILL_SPLIT = 1,    /* cut sequences into segments at checkpoint positions */
    KDA_PREFILL_PAIRED = 2,   /* two workgroups per chain: state-independent and state phases overlap */
    KDA_PREFILL_PAIRED_POLL_ONCE = 4, /* with KDA_PREFILL_PAIRED, for tests only: every wait between
                                         the two workgroups of a chain polls once before it gives up */
    KDA_PREFILL_CONV_DONE = 8         /* q, k, v as written by kda_project_inputs_conv: the conv and
                                         SiLU are done; bf16 activations only */
} kda_prefill_flags;

typedef struct {
    int32_t num_heads;   /* H: heads handled by this call (one GPU's share) */
    int32_t head_k;      /* dk */
    int32_t head_v;      /* dv */
    int32_t conv_width;  /* must be 4 */
    int32_t act_dtype;   /* kda_dtype of q, k, v, z, out and the conv state */
    float l2_eps;        /* eps inside the q/k L2 norm (1e-6 by convention) */
    float rms_eps;       /* eps inside the output RMSNorm (1e-6 by convention) */
    int32_t state_dtype; /* kda_dtype of the stored recurrent state (pools and
                            checkpoints); KDA_F32 (0) by default.  The state
                            math is fp32 either way.  With KDA_BF16 the state
                            is rounded to nearest bf16 (ties to even) wherever
                            it is stored -- after every decode step, at every
                            prefill checkpoint and at the prefill end -- and
                            computation continues from the rounded state, so
                            resuming from a checkpoint stays bit-identical in
                            the stored dtype.  [vLLM recipe
                            "moonshotai/Kimi-K3", section "AMD MI355X:
                            disaggregated prefill and decode": the worker
                            command keeps this state cache in bfloat16.] */
} kda_config;

/*
 * One decode step for B sequences, one token each, in ONE kernel launch.
 * [vLLM blog, "KDA prefill and decode": decode fuses the short convolution,
 *  the state update, the output gate and the normalisation instead of
 *  launching them separately; agentlenshq, "Fused Kernels and Metadata
 *  Optimization": one launch, no intermediate tensors, the state is read and
 *  written once.]
 *
 * q, k, v, z, g, beta: this step's inputs, layouts above with T = B.
 * state_pool, conv_pool: pools of num_slots slots; sequence b reads and
 *   updates slot slot[b] in place (state and conv state).
 * slot: [B] int32 device array.  Ids must be distinct within a call; an id
 *   outside [0, num_slots) makes the kernel skip that sequence and write NaN
 *   to its out row.
 * out: [B][H][dv] activation dtype.
 * B == 0 is a no-op.
 */
kda_status kda_decode_step(const kda_config* cfg, int32_t B,
                           const void* q, const void* k, const void* v, const void* z,
                           const float* g, const float* beta,
                           const float* conv_w, const float* norm_w,
                           void* state_pool, void* conv_pool, int32_t num_slots,
                           const int32_t* slot, void* out, void* stream);

/*
 * T decode tokens for each of B sequences in ONE launch, for the verify pass
 * of speculative decoding (K drafted tokens plus one).
 * [agentlenshq "vLLM Kimi K3 Support", section "Speculative Decoding with
 *  DSpark": the model is served with a drafting speculator; vLLM recipe
 *  "moonshotai/Kimi-K3", section "AMD MI355X: disaggregated prefill and
 *  decode": the decode worker drafts four tokens per step.]
 *
 * Inputs as kda_decode_step with a leading token axis: q, k, g [T][B][H][dk],
 *   v, z, out [T][B][H][dv], beta [T][B][H] (token t of sequence b at [t][b]).
 * The result equals T successive kda_decode_step calls bit for bit: the pool
 *   slot ends with the state and conv state after all T tokens.
 * token_state: NULL or [B][T][H][dk][dv] in the state dtype; token_conv: NULL
 *   or [B][T][H][2dk+dv][3] in the activation dtype.  When given they receive
 *   the state / conv state after every token, at slot b*T + t of a pool of
 *   B*T slots.  Rolling sequence b back to its first a tokens (1 <= a <= T) is
 *   then kda_resume from source slot b*T + a - 1 of those pools.
 * A sequence whose slot id is outside the pool gets NaN outputs for all T
 *   tokens and nothing written.  T >= 1; B == 0 is a no-op.
 */
kda_status kda_decode_multi(const kda_config* cfg, int32_t B, int32_t T,
                            const void* q, const void* k, const void* v, const void* z,
                            const float* g, const float* beta,
                            const float* conv_w, const float* norm_w,
                            void* state_pool, void* conv_pool, int32_t num_slots,
                            const int32_t* slot, void* out,
                            void* token_state, void* token_conv, void* stream);

/*
 * Chunked prefill of num_seqs packed sequences (chunk = 64 tokens).
 * [vLLM blog, "KDA prefill and decode": the prefill gathers each request's
 *  initial recurrent state in one operation; "The Hardest Part": a resumable
 *  state must exist at the exact prefix boundary; agentlenshq, "Agentic Cache
 *  Retention Policies": states are kept at fixed intervals and at prompt ends.]
 *
 * cu_seqlens: [num_seqs+1] int32 device array, cu_seqlens[0] == 0, non-
 *   decreasing, cu_seqlens[num_seqs] == total_tokens.  Sequence n owns packed
 *   tokens [cu_seqlens[n], cu_seqlens[n+1]).  Empty sequences are allowed.
 * start_pos: [num_seqs] int64 device array or NULL (all zero): the absolute
 *   position of each sequence's first token.  Chunks are aligned to absolute
 *   multiples of 64, so a sequence resumed at a multiple of 64 computes the
 *   same bits as the run that went straight through.
 * init_slot: [num_seqs] int32: slot of the initial state and conv state in
 *   the pools, or -1 for a zero state.
 * final_slot: [num_seqs] int32: slot that receives the final state and conv
 *   state, or -1 for none.  init_slot[n] == final_slot[n] (in place) is
 *   allowed; final slots must be distinct and must not be another sequence's
 *   init slot.
 * ckpt_interval: 0 = no checkpoints; otherwise a positive multiple of 64.
 *   Sequence n then writes a checkpoint at every absolute position p with
 *   p % ckpt_interval == 0 strictly inside (start, start+len), and at its end
 *   p = start+len (once if both); kda_num_checkpoints() gives the count.  Its
 *   j-th checkpoint goes to checkpoint slot ckpt_base[n] + j of ckpt_state /
 *   ckpt_conv (pools of num_ckpt_slots slots, same layout as the live pools).
 *   A checkpoint at p holds the state after the tokens before position p.
 * out: [total_tokens][H][dv] activation dtype.
 * workspace: device scratch of at least kda_prefill_workspace_bytes(...)
 *   bytes; its contents on entry do not matter.  Its first 4 bytes are the
 *   call's status word (int32): once the call has completed on its stream it
 *   holds the number of waits between paired workgroups that gave up (see
 *   KDA_PREFILL_PAIRED), 0 when every chain ran to its end.  It is always 0
 *   after a call without KDA_PREFILL_PAIRED; a call with num_seqs == 0
 *   launches nothing and leaves it untouched.
 * flags: 0, KDA_PREFILL_SPLIT or KDA_PREFILL_PAIRED (not both), and
 *   KDA_PREFILL_PAIRED_POLL_ONCE only together with KDA_PREFILL_PAIRED;
 *   KDA_PREFILL_CONV_DONE with any of them (bf16 activations).
 * KDA_PREFILL_CONV_DONE: q, k and v each point to two tensors back to back as
 *   kda_project_inputs_conv writes them (post-conv activations, then the raw
 *   inputs); the conv and SiLU are skipped and the raw inputs only feed the
 *   conv states of checkpoints and final slots.
 * KDA_PREFILL_SPLIT (needs ckpt_interval > 0).  Without it each
 *   (sequence, head) chain runs through its chunks in order in one workgroup,
 *   so a batch of few long sequences occupies few compute units.  With it,
 *   every sequence is cut at its interval checkpoint positions into segments
 *   that run in parallel.  The update is affine in the state (each token
 *   multiplies it by (I - b k k^T) Diag(exp g) and adds b k v^T), so a
 *   segment maps its initial state S to F S + G, where F is the state that
 *   the identity reaches with v = 0 and G the state that zero reaches; the
 *   segments' F and G are computed in parallel, a scan forms every segment's
 *   initial state in fp32, and the segments then run again from those states
 *   to produce their outputs.  The scan results are the interval checkpoints.
 *   About two and a half times the arithmetic of the unsplit run (each
 *   chunk's state-independent work twice, its state phase three times: G, F
 *   and the outputs), for parallelism over segments as well as sequences and
 *   heads; worth it when sequences x heads
 *   is well below the number of compute units [vLLM blog, introduction:
 *   contexts of up to one million tokens].  Results agree with an unsplit run
 *   to fp32 rounding.  A run resumed from one of its interval checkpoints with
 *   the same interval and flags reproduces it bit for bit; a continuation
 *   from a sequence end that is not an interval position agrees to rounding.
 * KDA_PREFILL_PAIRED: a grid of workgroups that are all resident at once
 *   (cooperative launch) schedules the (sequence, head) chains.  The longest
 *   chains get two workgroups each.  One computes every chunk's
 *   state-independent part (conv, norms, decays, the intra-chunk products
 *   and triangular inverses).  The other applies each chunk to the state and
 *   writes the outputs, checkpoints and final state; the chunks pass between
 *   them through a ring in the workspace, so the two parts of consecutive
 *   chunks overlap.  The other workgroups, and each pair once its chain is
 *   done, take the remaining chains one at a time from a queue, longest
 *   first.  How many chains to pair is decided on the device from the
 *   sequence lengths.  The results are bit for bit those of a call without
 *   the flag.  The workspace grows by the ring: three slots of about 142 KB
 *   per pair at dk = dv = 128, for up to min(sequences x heads, 256) pairs.
 *   On a device that cannot hold 16 such workgroups at once, the call runs
 *   as without the flag.  The launch needs its whole grid resident, so
 *   work running on the device at the same time can delay its start.  A
 *   paired call captured in a HIP graph replays bit for bit in the tests;
 *   every wait between the two workgroups of a chain is bounded, so a launch
 *   whose grid is not all resident cannot hang.  A wait that gives up counts
 *   in the status word; when it is the state-phase workgroup's, its chain's
 *   outputs from that chunk on, its final slot's state and the states of its
 *   checkpoints still due (this head's) are written as NaN, so none of them
 *   passes for a valid state.  KDA_PREFILL_PAIRED_POLL_ONCE makes every such
 *   wait poll only once, so tests can drive this path without a stalled
 *   partner.
 * Gates: any g <= 0, including -inf.  Within a chunk the pairwise decays
 *   exp(Gam_t - Gam_s) (Gam the running sum of g) are formed through the
 *   chunk's middle row while every channel's decay over each half of the
 *   chunk stays above -80, and from sums over 16-token blocks otherwise (a
 *   slower path, exact pairs within a block); log-decays below -30 then count
 *   as -30 (exp(-30) = 9.4e-14: what they let through is below the fp32
 *   resolution of the state).  Which path a chunk takes depends only on its
 *   own gates, so resumes stay bit-identical.
 */
kda_status kda_prefill_varlen(const kda_config* cfg, int32_t num_seqs, int64_t total_tokens,
                              const int32_t* cu_seqlens, const int64_t* start_pos,
                              const void* q, const void* k, const void* v, const void* z,
                              const float* g, const float* beta,
                              const float* conv_w, const float* norm_w,
                              void* state_pool, void* conv_pool, int32_t num_slots,
                              const int32_t* init_slot, const int32_t* final_slot,
                              int32_t ckpt_interval, void* ckpt_state, void* ckpt_conv,
                              int32_t num_ckpt_slots, const int32_t* ckpt_base, int32_t flags,
                              void* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation:
 * kda_prefill_varlen with the same arguments and results, its workspace taken
 * from a static device buffer of KDA_STATIC_WORKSPACE_BYTES instead of an
 * argument.  The library holds one such buffer on every device it runs on
 * until the process ends, and this call allocates nothing.
 *
 * Limit: the call must fit the buffer, i.e. kda_prefill_workspace_bytes(cfg,
 *   num_seqs, total_tokens, ckpt_interval, flags) <= KDA_STATIC_WORKSPACE_BYTES;
 *   otherwise it returns KDA_ERR_WORKSPACE and launches nothing.  That holds
 *   for the one-workgroup launch of up to about two million sequences, for
 *   KDA_PREFILL_PAIRED with up to 153 (sequence, head) chains at dk = dv = 128
 *   (its ring takes 436 KB per chain), and for KDA_PREFILL_SPLIT with up to
 *   about 340 (possible segment, head) pairs at dk = dv = 128 (192 KB each;
 *   a call has 2 num_seqs + total_tokens / ckpt_interval possible segments).
 * Sharing: every call on a device uses that device's one buffer, and the
 *   buffer keeps the last call's contents (each call initialises what it
 *   reads).  Calls whose kernels overlap in time on one device -- on
 *   different streams, or from different host threads -- race on it and give
 *   undefined results; serialise them (one stream, or events).
 * The status word of the workspace (see kda_prefill_varlen) is not visible to
 *   the caller; a chain whose paired wait gave up still shows NaN outputs.
 */
#define KDA_STATIC_WORKSPACE_BYTES (64LL << 20)
kda_status kda_prefill_varlen_static(const kda_config* cfg, int32_t num_seqs, int64_t total_tokens,
                                     const int32_t* cu_seqlens, const int64_t* start_pos,
                                     const void* q, const void* k, const void* v, const void* z,
                                     const float* g, const float* beta,
                                     const float* conv_w, const float* norm_w,
                                     void* state_pool, void* conv_pool, int32_t num_slots,
                                     const int32_t* init_slot, const int32_t* final_slot,
                                     int32_t ckpt_interval, void* ckpt_state, void* ckpt_conv,
                                     int32_t num_ckpt_slots, const int32_t* ckpt_base, int32_t flags,
                                     void* out, void* stream);

/*
 * Input projections of the layer for T tokens in one bf16 MFMA GEMM:
 * y = x W^T, routed by rows of W to q, k (H dk each), v, z (H dv each), the
 * decay gate (H dk: g = -softplus(y)) and beta (H: beta = sigmoid(y)).
 * [vLLM blog, "KDA prefill and decode": the input projections are fused around
 *  the recurrence.  The pages give no gate parameterisation; -softplus and the
 *  logistic function of a linear pre-activation are the readings used here.]
 *
 * x: [T][Dm] bf16; w: [N][Dm] bf16 with N = H (3 dk + 2 dv) + H, rows in the
 *   order q, k, v, z, g, beta (each head's channels consecutive).
 * q, k: [T][H][dk], v, z: [T][H][dv] bf16 (RNE); g: [T][H][dk] fp32;
 *   beta: [T][H] fp32 -- exactly the inputs kda_prefill_varlen and
 *   kda_decode_step take.  Accumulation in fp32.
 * Requires act_dtype == KDA_BF16 and Dm a positive multiple of 64, at most
 * 4194304.
 */
kda_status kda_project_inputs(const kda_config* cfg, int32_t T, int32_t Dm,
                              const void* x, const void* w,
                              void* q, void* k, void* v, void* z, float* g, float* beta,
                              void* stream);

/*
 * The input projections with the causal conv fused into the GEMM's epilogue:
 * the front end of a chunked prefill over num_seqs packed sequences.
 * [vLLM blog, "KDA prefill and decode": the input projections and the causal
 *  convolution are fused around the recurrence.]
 *
 * Arguments as kda_project_inputs, plus cu_seqlens ([num_seqs+1] int32
 * device array as for kda_prefill_varlen, describing the T packed tokens of
 * x), conv_w ([H][2dk+dv][4] fp32) and the initial conv states: sequence n's
 * left context is conv_pool[init_slot[n]] ([num_slots][H][2dk+dv][3] bf16,
 * index 2 = the token just before the sequence), or zero when init_slot is
 * NULL or init_slot[n] is -1 (an id outside the pool counts as -1).
 * q, k and v each point to TWO tensors back to back ([2][T][H][dk] for q
 * and k, [2][T][H][dv] for v, bf16):
 *   first  the activations after the conv: RNE_bf16(SiLU(w3 r_t + w2 r_{t-1}
 *          + w1 r_{t-2} + w0 r_{t-3})), r the raw projections rounded to bf16
 *          (rows before a sequence's first token from its left context),
 *          the value kda_prefill_varlen forms in fp32 from the raw inputs;
 *   second the raw projections r themselves (what conv states hold).
 * z, g and beta as kda_prefill_varlen takes them.  Pass q, k, v, z, g, beta
 * to kda_prefill_varlen with KDA_PREFILL_CONV_DONE (same cu_seqlens, and the
 * same initial conv states as its init_slot gives): it then skips the conv,
 * and its checkpoints and final conv states hold the raw inputs as without
 * the flag.  The one difference from the unfused pair kda_project_inputs +
 * kda_prefill_varlen is the rounding of the post-conv activations to bf16.
 * The GEMM runs in tiles of 256 rows that overlap by 3 (each recomputes the
 * conv's left context of its first row): 1.2% more MFMA work.
 */
kda_status kda_project_inputs_conv(const kda_config* cfg, int32_t num_seqs, int32_t T, int32_t Dm,
                                   const int32_t* cu_seqlens, const void* x, const void* w,
                                   const float* conv_w, const void* conv_pool, int32_t num_slots,
                                   const int32_t* init_slot,
                                   void* q, void* k, void* v, void* z, float* g, float* beta,
                                   void* stream);

/*
 * Output projection of the layer for T tokens in one bf16 MFMA GEMM:
 * y = o W_o^T, from the layer's gated, normalised output back to the model
 * width.  [The pages name no output projection; a linear map back to the
 *  model width is the plain reading of a layer in the residual stream.]
 *
 * o: [T][H][dv] bf16 (the `out` of kda_prefill_varlen / kda_decode_step);
 * w_o: [Dm][H dv] bf16; y: [T][Dm] bf16 (RNE).  Accumulation in fp32.
 * Requires act_dtype == KDA_BF16 and H dv a multiple of 64 (at most
 * 4194304); o and w_o 16-byte aligned, y 2-byte aligned.  Any Dm >= 1.
 */
kda_status kda_project_output(const kda_config* cfg, int32_t T, int32_t Dm,
                              const void* o, const void* w_o, void* y, void* stream);

/*
 * Copy n (state, conv state) slot pairs from the live pools to checkpoint
 * slots: ckpt[dst_ckpt[i]] = pool[src_slot[i]], bit for bit, all heads.
 * [vLLM blog, "The Hardest Part": the state registered at a boundary is kept
 *  apart from the request that goes on extending it.]
 * Ids outside their pool are skipped.  Destinations must be distinct.
 */
kda_status kda_state_checkpoint(const kda_config* cfg, int32_t n,
                                const void* state_pool, const void* conv_pool, int32_t num_slots,
                                const int32_t* src_slot,
                                void* ckpt_state, void* ckpt_conv, int32_t num_ckpt_slots,
                                const int32_t* dst_ckpt, void* stream);

/*
 * Copy-on-write resume: pool[dst_slot[i]] = ckpt[src_ckpt[i]], bit for bit.
 * The checkpoint stays untouched, so one checkpoint can seed many slots.
 * [vLLM blog, "The Hardest Part": a hit on a cached boundary copies the
 *  cached state into a private destination before the request extends it,
 *  and reuse within the same step waits until the copy is safe.]
 * Ordering: the copy is enqueued on `stream`; a kernel that reads a
 * destination slot must be enqueued after it on the same stream (or wait on
 * an event recorded after it).  Ids outside their pool are skipped.
 */
kda_status kda_resume(const kda_config* cfg, int32_t n,
                      const void* ckpt_state, const void* ckpt_conv, int32_t num_ckpt_slots,
                      const int32_t* src_ckpt,
                      void* state_pool, void* conv_pool, int32_t num_slots,
                      const int32_t* dst_slot, void* stream);

/* Workspace bytes kda_prefill_varlen needs for these sizes, checkpoint
 * interval and flags (0 on an error; kda_last_error() then says why).  With
 * KDA_PREFILL_SPLIT it holds, per possible segment (at most 2 num_seqs +
 * total_tokens / ckpt_interval) and head, three dk x dv fp32 matrices; with
 * KDA_PREFILL_PAIRED, the ring of the scheduled launch (three slots per
 * pair, for min(num_seqs x heads, 256) pairs), its counters and its queue. */
size_t kda_prefill_workspace_bytes(const kda_config* cfg, int32_t num_seqs, int64_t total_tokens,
                                   int32_t ckpt_interval, int32_t flags);

/* Number of checkpoints kda_prefill_varlen writes for one sequence: the
 * multiples of interval strictly inside (start, start+len) plus its end; 0
 * when interval <= 0 or len <= 0.  Host function. */
int64_t kda_num_checkpoints(int64_t start, int64_t len, int32_t interval);

/* Message of the last error on this thread ("" if none). */
const char* kda_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
