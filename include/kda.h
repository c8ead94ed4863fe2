/*
 * kda.h -- C ABI of libkda: Kimi Delta Attention (KDA) multi-token recurrent
 * prefill on AMD Instinct MI355X (gfx950).
 *
 * What one call computes.  For every sequence n of a fixed or packed batch and
 * every head h, independently, starting from an fp32 K x V state S (K = V =
 * 128, row d = key channel; the initial state, or zeros) and for each token t
 * of the sequence in order:
 *
 *   S   <- Diag(exp(g_t)) S                     decay per key channel, g_t <= 0
 *   S   <- S + beta_t k_t (v_t - S^T k_t)^T      delta-rule rank-1 correction
 *   o_t <- scale * S^T q_t                        read-out of the updated state
 *
 * This is Kimi Delta Attention as used by Kimi Linear: a fixed-size recurrent
 * state per head (FlashKDA page, item description), with the prefill contract
 * of lmdeploy PR #5050 (Modification: BF16 inputs, K/V dimensions of 128, FP32
 * recurrent state, gate lower bound in [-5, 0], checkpoint export at a
 * requested position) and of FlashInfer PR #4262 "cake_kda" (Dispatch
 * contract: fixed [B, T, H, 128] or packed inputs with cu_seqlens).  q and k
 * are taken as given (callers L2-normalise them beforehand), g is a finished
 * natural-log decay and beta an already-activated strength in [0, 1].
 *
 * The device computes the chunk-parallel form of the same recurrence (chunks
 * of 64 tokens aligned to each sequence start), so results equal the token
 * recurrence up to floating-point rounding.
 *
 * Layouts (all row-major, last index fastest, all buffers device memory):
 *   q, k, v        bf16  [T_total, H, 128]
 *   g              fp32  [T_total, H, 128]   lower_bound <= g <= 0
 *   beta           fp32  [T_total, H]
 *   cu_seqlens     int32 [N + 1] (int64 with kda_problem.cu_seqlens_int64), or
 *                  NULL for a fixed batch of N sequences of T_total / N tokens.  Contract when given (not checked on the
 *                  device, as in lmdeploy PR #5050, Modification: offset values
 *                  stay the caller's responsibility so nothing synchronises):
 *                  cu[0] = 0, cu[N] = T_total, non-decreasing.
 *   initial_state  fp32  [N, H, 128, 128] (K x V), or NULL for zeros
 *   out            bf16  [T_total, H, 128]; may be exactly v (same pointer)
 *   final_state    fp32  [N, H, 128, 128], or NULL; may be exactly
 *                  initial_state (in-place update, FlashInfer PR #4262,
 *                  Physical schedules and true in-place state update)
 *   ckpt_offsets   int32 [N, C] (C = kda_problem.ckpt_per_seq, 1 by default),
 *                  or NULL: ckpt_offsets[n, c] = number of tokens of sequence
 *                  n consumed when its state is exported into slot c (0
 *                  exports the initial state, L_n the final state).  A
 *                  sequence's offsets are taken in order; one is honoured when
 *                  it lies in [0, L_n] and is not below the previous honoured
 *                  one.  The others export nothing and leave their slot
 *                  untouched, so -1 pads a shorter list (e.g. periodic
 *                  checkpoints every n tokens of sequences of unequal length).
 *   ckpt_state     fp32  [N, C, H, 128, 128] caller-owned, contiguous; NULL iff
 *                  ckpt_offsets is NULL; must not overlap either state buffer.
 *
 * Ownership and streams: every buffer belongs to the caller; the library
 * allocates nothing, keeps no pointer after returning and holds no state
 * between calls.  All work is enqueued on `stream` with no host
 * synchronisation and no device-to-host copy, so a call can be captured in a
 * HIP graph without warm-up.  Errors are detected on the host before anything
 * is enqueued; device-resident values (cu_seqlens, offsets, g) are not read on
 * the host.  A zero-length sequence keeps its initial state bit for bit.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = -1,      /* bad sizes, NULL where required, bad scalar */
  KDA_ERR_UNSUPPORTED = -2,      /* head dims other than 128, unknown variant */
  KDA_ERR_ALIGNMENT = -3,        /* a pointer not 16-byte aligned */
  KDA_ERR_OVERLAP = -4,          /* buffers overlap other than the allowed exact aliases */
  KDA_ERR_WORKSPACE_TOO_SMALL = -5,
  KDA_ERR_TOO_LARGE = -6,        /* T_total * H * 128 exceeds 2^31 - 1 */
  KDA_ERR_HIP = -7,              /* a HIP runtime call or launch failed */
  KDA_ERR_SCRATCH_TOO_SMALL = -8 /* kda_prefill_noalloc: the problem's workspace exceeds
                                    KDA_NOALLOC_SCRATCH_BYTES */
} kda_status;

typedef enum {
  KDA_VARIANT_AUTO = 0,          /* pick the schedule from a table keyed on the CU count and
                                    the shape the host knows (N, H, T_total / N): the one-launch
                                    schedule for short sequences (a mean of at most 64 tokens)
                                    whose workgroups all fit on the device at once, else the
                                    two-launch schedule when the workspace holds it, with four
                                    workgroups per (sequence, head) when they all fit at once
                                    and the workspace is past 176 MiB, else two */
  KDA_VARIANT_DECOMP = 1,        /* two launches through the workspace: a chunk-parallel
                                    prepare, then the recurrence (FlashInfer PR #4633,
                                    Description: the "decomp" variant) */
  KDA_VARIANT_FUSED = 2          /* one launch: chunk preparation and recurrence per workgroup
                                    (same page: the "fused" variant); needs no workspace */
} kda_variant;

typedef struct {
  int32_t num_seqs;          /* N >= 1 (fixed layout: the batch size B) */
  int64_t total_tokens;      /* T_total >= 0 (fixed layout: B * T) */
  int32_t num_heads;         /* H >= 1, shared by q, k and v */
  int32_t head_dim_k;        /* must be 128 */
  int32_t head_dim_v;        /* must be 128 */
  float scale;               /* read-out scale, finite (typically 1/sqrt(128)) */
  float gate_lower_bound;    /* caller's promise g >= bound; must lie in [-5, 0] */
  int32_t variant;           /* kda_variant */
  int32_t value_split;       /* 0 = automatic, else workgroups per (sequence, head), each
                                owning 128/value_split columns of the state: 2 or 4 for
                                FUSED, 1, 2, 4 or 8 for DECOMP (FlashInfer PR #4262,
                                Physical schedules: value rows split over CTAs) */
  int32_t stages;            /* DECOMP only (0 otherwise): which of its two launches to
                                enqueue.  0 = both.  KDA_STAGE_PREPARE = only the chunk-
                                parallel prepare, which fills the workspace.
                                KDA_STAGE_RECURRENCE = only the recurrence, which reads a
                                workspace that an earlier PREPARE call filled from the same
                                inputs and problem (the caller's contract, not checked) */
  int32_t ckpt_per_seq;      /* C, checkpoint offsets per sequence, 0..64 (0 means 1).
                                ckpt_offsets is then int32 [N, C] and ckpt_state fp32
                                [N, C, H, 128, 128]; see kda_prefill */
  int32_t state_dtype;       /* kda_state_dtype of initial_state, final_state and
                                ckpt_state (same layouts, 2-byte elements for BF16).
                                The recurrence itself always carries fp32; a BF16 state
                                is widened on load and rounded to nearest even on store
                                (the BF16 state of FlashInfer PR #4262's benchmark) */
  int32_t prologue;          /* kda_prologue flags, 0 = none: inputs as given.  Both
                                schedules apply them */
  int32_t cu_seqlens_int64;  /* 0: cu_seqlens holds int32 offsets; 1: int64 offsets.  Both are
                                read as they are on the device (FlashInfer PR #4262, Dispatch
                                contract: packed offsets come as int32 or int64, and a captured
                                graph takes them with no conversion) */
  const int32_t* seq_order;  /* packed layout only, optional: device int32 [N], the order in
                                which the two-launch schedule's recurrence takes the sequences
                                (FlashInfer PR #4262, Dispatch contract: an optional int32
                                seq_order orders packed sequences for tail utilisation).  NULL:
                                longest first (up to 1024 sequences), chosen on the device.  It
                                must hold a permutation of 0..N-1 with N <= 65536; the plan
                                launch checks that on the device and takes the identity order
                                when it does not.  Results do not depend on the order.  The
                                fixed layout and FUSED (whose workgroups all run at once when
                                AUTO picks it) do not use it */
  int32_t chain_parts;       /* two-launch schedule: pieces each (sequence, head)'s chain of
                                segments is cut into, 0..KDA_MAX_CHAIN_PARTS.  0 = automatic
                                (kda_plan reports the choice), 1 = no split.  With P >= 2 the
                                recurrence runs as two launches: the first runs piece 0 from
                                the initial state and pieces 1..P-2 both from a zero state and
                                from the identity with V = 0 (the state update is affine in the
                                state, so these two give each piece's map S -> T S + B); a scan
                                composes the maps into each piece's incoming state; the second
                                runs pieces 1..P-1 from those states with outputs and
                                checkpoints.  It trades about 3x the recurrence's work for a
                                chain P times shorter, for problems with too few pairs to fill
                                the device (FlashInfer PR #4633, Performance: the B1 T8192 row
                                is the recurrence's chain alone).  Results equal the unsplit
                                recurrence's up to rounding.  FUSED takes 0 or 1 only; with
                                AUTO, 2 or more selects DECOMP (as value_split 1 and 8 do) */
} kda_problem;

#define KDA_MAX_CHAIN_PARTS 16

/* Input prologue, done in the kernels before anything else reads q, k or
 * beta (FlashInfer PR #4262, Dispatch contract, lists kernels with q/k
 * L2-normalisation inside and beta as a logit). */
typedef enum {
  KDA_PROLOGUE_QK_L2NORM = 1,  /* q_t, k_t divided by their Euclidean norms over the 128
                                  channels, per token and head (a zero vector stays zero) */
  KDA_PROLOGUE_BETA_LOGIT = 2  /* beta holds logits: beta_t = 1 / (1 + exp(-beta_t)) */
} kda_prologue;

typedef enum {
  KDA_STATE_F32 = 0,         /* fp32 states (the contract the pages fix) */
  KDA_STATE_BF16 = 1         /* bf16 states */
} kda_state_dtype;

enum { KDA_STAGE_PREPARE = 1, KDA_STAGE_RECURRENCE = 2 };

/* Bytes of caller workspace kda_prefill needs for this problem (host only, no
 * device access).  The two-launch schedule's prepare and recurrence share one
 * caller-owned scratch arena, which is what makes graph capture possible
 * (FlashInfer PR #4633, Description: decomp shares a scratch arena between its
 * two launches; capture goes through a caller-owned workspace).  lmdeploy PR
 * #5050, Modification, has the backend allocate its workspace; here the caller
 * does, so that nothing is allocated inside a call.  FUSED needs none (0).  DECOMP, and AUTO so that it may
 * pick DECOMP, need a header of 2 N + 1 int32 rounded up to 256 bytes plus
 * 60,416 bytes per (segment slot, head), with floor(T_total / 64) + N + N C
 * segment slots (C = ckpt_per_seq, at least 1): about 0.94 KiB per
 * token-head.  A chain split of P pieces adds 3 x 64 KiB per (sequence, head,
 * piece), with P = chain_parts when given, else, for AUTO and DECOMP, the
 * most pieces AUTO may pick: min(16, 1 + floor(128 / (N H)),
 * floor(ceil((T_total / N) / 64) / 8)) when that is at least 3 (else none).
 * A smaller workspace that still holds the slots runs AUTO unsplit.  The
 * workspace is scratch:
 * it carries nothing between calls, may be reused by any later call on the
 * same stream, and must not be used by two calls in flight at once. */
kda_status kda_prefill_workspace_size(const kda_problem* p, size_t* bytes);

/* Host-side argument checks of kda_prefill without launching anything: sizes,
 * the K = V = 128 and gate-bound contract, NULL rules, 16-byte alignment,
 * overlap (only out == v and final_state == initial_state may alias, and
 * only exactly), workspace size and the INT32 bound on T_total * H * 128
 * (FlashInfer PR #4633, Description: the flat output is bounded on the host).
 * Pointers are compared, never dereferenced, so host addresses may be used. */
kda_status kda_validate(const kda_problem* p, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const void* cu_seqlens,
                        const float* initial_state, const void* out, const float* final_state,
                        const int32_t* ckpt_offsets, const float* ckpt_state,
                        const void* workspace, size_t workspace_bytes);

/* Enqueue one prefill on `stream` (a hipStream_t; NULL = the null stream).
 * q, k, v, out are bf16 bit patterns (uint16_t).  Returns KDA_OK once the work
 * is enqueued; any other status means nothing was enqueued, except
 * KDA_ERR_HIP, which reports a failed launch. */
kda_status kda_prefill(const kda_problem* p, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const float* g, const float* beta,
                       const void* cu_seqlens, const float* initial_state, uint16_t* out,
                       float* final_state, const int32_t* ckpt_offsets, float* ckpt_state,
                       void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * prefill as kda_prefill, with the DECOMP workspace taken from a static device
 * buffer of KDA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends (its device address is looked up on the first
 * call on each device).  The call allocates nothing.
 *   - Sizes: a problem whose workspace (kda_prefill_workspace_size) exceeds
 *     KDA_NOALLOC_SCRATCH_BYTES returns KDA_ERR_SCRATCH_TOO_SMALL before
 *     anything is enqueued, unless its variant is KDA_VARIANT_FUSED (no
 *     workspace).  With AUTO the schedule is the one kda_plan names.
 *   - Sharing: all calls on one GPU share that GPU's buffer.  It keeps the last
 *     call's contents, and nothing in it needs to start at zero (the prepare
 *     launch writes every byte the recurrence reads).  Calls that overlap in
 *     time on one GPU (two streams, or two threads) race on it; serialise them.
 *   - Everything else (arguments, errors, aliasing, streams) is as kda_prefill. */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20)
kda_status kda_prefill_noalloc(const kda_problem* p, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const float* g, const float* beta,
                               const void* cu_seqlens, const float* initial_state, uint16_t* out,
                               float* final_state, const int32_t* ckpt_offsets, float* ckpt_state,
                               void* stream);

/* ---------------------------------------------------------------------------
 * State-pool decode.  A serving step advances each of N requests by T tokens
 * (T = 1: decode; T > 1: e.g. verifying T draft tokens) from the fp32 state
 * its index names in a pool, and writes the state back in place.  The
 * per-request pool index follows the state pool / ssm_state_indices of the
 * sglang KDA decode backend (FlashInferKDAKernel page); FlashInfer PR #4262
 * (Description) names decode (T = 1) and state-pool features as the
 * counterpart of the prefill.  For request n with i = state_indices[n] in
 * [0, pool_size) and every head h, starting from S = pool[i, h], each token t
 * of the request applies the recurrence stated at the top of this file and
 * the final S is stored to pool[i, h].  An index outside [0, pool_size)
 * (such as -1 for an empty batch slot) leaves the pool untouched and gives
 * zero outputs.
 *
 * Layouts (device memory):
 *   q, k, v     bf16 [N * T, H, 128]   (request-major: token t of request n is row n * T + t)
 *   g           fp32 [N * T, H, 128],  lower_bound <= g <= 0
 *   beta        fp32 [N * T, H]
 *   state_pool  fp32 [pool_size, H, 128, 128] (K x V), read and written in place
 *   state_indices int32 [N]; non-negative entries must be distinct (two
 *               requests on one state race; not checked on the device)
 *   out         bf16 [N * T, H, 128]; may be exactly v
 * The update runs token by token in fp32 (no chunking).  Errors are detected
 * on the host before anything is enqueued; nothing is allocated. */
typedef struct {
  int32_t num_seqs;          /* N >= 0 requests */
  int32_t tokens_per_seq;    /* T >= 1 tokens per request */
  int32_t num_heads;         /* H >= 1 */
  int32_t head_dim_k;        /* must be 128 */
  int32_t head_dim_v;        /* must be 128 */
  float scale;               /* read-out scale, finite */
  float gate_lower_bound;    /* caller's promise g >= bound; must lie in [-5, 0] */
  int64_t pool_size;         /* states in the pool, >= 1 */
  int32_t prologue;          /* kda_prologue flags, as for kda_prefill */
  int32_t state_dtype;       /* kda_state_dtype of the pool and of a verify's state
                                trace: fp32, or bf16 (same layouts, 2-byte elements,
                                passed through the same pointer types).  The tokens
                                run in fp32 from the widened state; a bf16 state is
                                rounded to nearest even once, when it is stored (the
                                BF16 state of FlashInfer PR #4262's benchmark) */
} kda_decode_problem;

/* Host-side checks of kda_decode without launching: sizes, NULL rules,
 * 16-byte alignment, overlap (only out == v may alias, exactly), and the
 * INT32 bound on N * T * H * 128.  Pointers are never dereferenced. */
kda_status kda_decode_validate(const kda_decode_problem* p, const void* q, const void* k,
                               const void* v, const float* g, const float* beta,
                               const float* state_pool, const int32_t* state_indices,
                               const void* out);

/* Enqueue one decode step on `stream` (a hipStream_t; NULL = the null
 * stream).  Same status convention as kda_prefill. */
kda_status kda_decode(const kda_decode_problem* p, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const float* g, const float* beta, float* state_pool,
                      const int32_t* state_indices, uint16_t* out, void* stream);

/* Speculative verify, then commit or advance.  FlashInfer PR #4262 (upstream
 * recurrent-KDA comparison) says speculative decode has different checkpoint /
 * state semantics from decode, and its dispatch contract names accepted-token
 * features; lmdeploy PR #5050 (Modification) keeps a ring of states for its
 * MTP decode kernels; none of them defines the semantics.  Reading taken:
 * verifying T draft tokens per request runs the decode recurrence over all T
 * (outputs for every position, as kda_decode) but leaves the pool as it is;
 * once the caller knows how many drafts each request accepted, the pool takes
 * the state after that accepted prefix.  Two ways to get there:
 *   - a trace: the verify stores the state after every token and a commit
 *     copies the accepted one (N T H x 64 KiB of trace; the intermediate
 *     states stay available to the caller);
 *   - a recompute: the verify stores no state and an advance runs the accepted
 *     prefix again from the pool, with no outputs (no trace; the pool's state
 *     is read twice and written once).
 *   kda_decode_verify: as kda_decode with the pool only read, plus
 *     state_trace fp32 [N, T, H, 128, 128] (device, caller-owned) or NULL (no
 *     trace): state_trace[n, t] = the state of request n after its first t + 1
 *     tokens.  A request with no pool index gives zero outputs and leaves its
 *     trace rows untouched.  state_trace must not overlap any other buffer.
 *   kda_decode_commit: for every request n with a pool index and
 *     1 <= accepted[n] <= T (accepted: device int32 [N], e.g. written by the
 *     sampler, so nothing synchronises), copies state_trace[n, accepted[n] - 1]
 *     into pool[state_indices[n]]; other requests (accepted[n] = 0: every draft
 *     rejected) keep their pool state.  Values in accepted are the caller's
 *     contract, as offsets are; out-of-range ones change nothing.
 *   kda_decode_advance: the same inputs as the verify (all T tokens' q, k, v,
 *     g, beta), no outputs: request n's pool state advances by its first
 *     accepted[n] tokens (accepted as for the commit; 0 or out of range leaves
 *     it as it is).  The pool is written in place and must not overlap the
 *     inputs, the indices or accepted.
 * After a verify, commit or advance with accepted[n] = T leaves the pool bit
 * for bit as kda_decode would have, and advance with any accepted[n] leaves it
 * bit for bit as the commit of the traced state does.  All three check their
 * arguments on the host first, as kda_decode. */
kda_status kda_decode_verify(const kda_decode_problem* p, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const float* g, const float* beta,
                             const float* state_pool, const int32_t* state_indices, uint16_t* out,
                             float* state_trace, void* stream);
kda_status kda_decode_commit(const kda_decode_problem* p, float* state_pool,
                             const int32_t* state_indices, const float* state_trace,
                             const int32_t* accepted, void* stream);
kda_status kda_decode_advance(const kda_decode_problem* p, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const float* g, const float* beta, float* state_pool,
                              const int32_t* state_indices, const int32_t* accepted, void* stream);

/* Static string for a status code (a kda_status value; any other int gives
 * "unknown status").  Errors are reported, never retried or rerouted through
 * another path (lmdeploy PR #5050, Modification: native execution errors are
 * propagated), and argument errors are found before anything is enqueued
 * (same passage: requests fail before any state is touched). */
const char* kda_status_string(int status);

/* Schedule, workgroups per (sequence, head) and chain pieces (1 = no split;
 * chain_parts may be NULL) kda_prefill would use for this problem on the
 * current device, given a workspace of at least kda_prefill_workspace_size
 * bytes (host only; reads the device's CU count).  The choice comes from a
 * table of measured rows keyed on the compute-unit count, not on the device's
 * name (FlashInfer PR #4633, Description: neither the two-launch nor the
 * one-launch kernel is faster everywhere, so a table keyed on SM count picks
 * per call, and a query reports the choice).  value_split is the count of the
 * unsplit recurrence and of the chain split's second launch; with value_split
 * 0 in the problem, the split's first launch (twice the workgroups) may run
 * with fewer per (sequence, head), from the same cost table. */
kda_status kda_plan(const kda_problem* p, int32_t* variant, int32_t* value_split,
                    int32_t* chain_parts);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
