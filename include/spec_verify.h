/*
 * spec_verify.h - batched speculative-sampling verifier for AMD MI355X (gfx950).
 *
 * One call verifies B rows of K draft tokens against one target pass:
 *
 *   - The target scored the prefix extended by the drafts in a single pass,
 *     so it provides K+1 next-token distributions per row: position i is
 *     conditioned on drafts d_0..d_{i-1}, position K is the bonus position
 *     ("Speculative decoding: memverifikasi token draft sebelum diterima",
 *     subsection "Draft mengubah tebakan serial menjadi batch verifikasi").
 *   - Both logit sets are turned into probabilities by softmax(l / T), the
 *     temperature acting at the verification gate (RheoSampling 2026,
 *     section 7).  The draft may first be cut to its topk_draft largest
 *     logits, the rest set to -inf, ties at the cut to the lowest id
 *     (RheoSampling 2026, section 3).
 *   - Draft d_i is accepted when u_i < min(1, p_i(d_i) / q_i(d_i)), evaluated
 *     as u_i * q < p; the first rejection ends the committed prefix
 *     (RheoSampling 2026, section 4, step 1; "Speculative decoding: ...",
 *     subsection "Penolakan memendekkan pekerjaan speculative yang berguna").
 *   - After a rejection at position n the final token is drawn from
 *     norm(max(0, p_n - q_n)); if all K drafts are accepted it is drawn from
 *     the bonus position p_K (RheoSampling 2026, section 4, step 3).  The
 *     draw is an inverse CDF in ascending token id with uniform u_K: the
 *     smallest x whose cumulative weight exceeds u_K * (total weight).
 *   - A row with T <= 0 is verified greedily: drafts are accepted while they
 *     equal the target's argmax (lowest id among equal maxima), and the
 *     target's argmax at the first mismatch (or at the bonus position) is
 *     emitted ("Speculative decoding: ...", subsection "Semantik penerimaan
 *     bergantung pada algoritma decoding").  Uniforms and draft logits of
 *     such rows are not read.
 *
 * All pointers are device pointers owned by the caller.  Inputs are read
 * only; outputs are fully overwritten.  The library allocates nothing, keeps
 * no mutable global state other than spec_verify_noalloc's static scratch,
 * and never synchronises: every call only enqueues
 * at most three kernels on `stream` (no memory set or copy), so a call can
 * be captured in a HIP graph and replayed; outputs are valid once the caller
 * has synchronised that stream.  Calls on different workspaces are
 * reentrant.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of both logit tensors. */
typedef enum { SV_BF16 = 0, SV_F32 = 1 } sv_dtype;

/* Return codes.  No call prints, throws or aborts. */
typedef enum {
  SV_OK = 0,
  SV_ERR_ARG = 1,          /* bad scalar or a NULL pointer that is required      */
  SV_ERR_WORKSPACE = 2,    /* *workspace_bytes smaller than the size required    */
  SV_ERR_UNSUPPORTED = 3,  /* 0 < topk_draft < V with topk_draft > SV_MAX_TOPK, or */
                           /* K > SV_MAX_K                                        */
  SV_ERR_HIP = 4,          /* a kernel launch failed (hipGetLastError)           */
  SV_ERR_SCRATCH = 5       /* spec_verify_noalloc: the shape needs more scratch  */
                           /* than SV_SCRATCH_BYTES                              */
} sv_status;

#define SV_MAX_TOPK 1024
#define SV_MAX_K 64
#define SV_MAX_NODES 64
/* Size of spec_verify_noalloc's static device scratch (per GPU). */
#define SV_SCRATCH_BYTES (32u << 20)

/*
 * spec_verify - verify B rows; see the description at the top of this file.
 *
 * target_logits  [B, K+1, V] device, dtype, row-major contiguous.
 * draft_logits   [B, K, V]   device, dtype, row-major contiguous; may be NULL
 *                when K == 0.
 * draft_tokens   [B, K] int32 device; may be NULL when K == 0.  A token outside
 *                [0, V) has p = q = 0 and is rejected.
 * uniforms       [B, K+1] float32 device, each in [0, 1).  u[b][i] (i < K)
 *                drives the acceptance test at position i; u[b][K] drives the
 *                final (correction or bonus) draw.
 * temperature    [B] float32 device; T <= 0 (or NaN) selects greedy for the row.
 * B >= 1, K in [0, SV_MAX_K], V >= 1.
 * topk_draft     0 or >= V: dense draft; otherwise keep the topk_draft largest
 *                draft logits per position (at most SV_MAX_TOPK).
 * dtype          sv_dtype of both logit tensors.
 * out_tokens     [B, K+1] int32 device: accepted drafts, the final token,
 *                then -1 padding.
 * num_accepted   [B] int32 device: number of accepted drafts, 0..K.  A row
 *                whose internal hand-off between work-groups did not complete
 *                within 100 ms (it completes in microseconds in any correct
 *                launch; the bound only guarantees termination) gets -1 here
 *                and -1 in every out_tokens slot.
 * workspace      device scratch of at least *workspace_bytes bytes, 256-byte
 *                aligned, zero-filled before its first use with a given
 *                shape (B, K, V, topk_draft, dtype), e.g. by hipMemset to 0.
 *                Every call leaves the regions its shape's layout needs
 *                zeroed again (its counters return to zero), so calls of the
 *                same shape can reuse it without clearing; a call of another
 *                shape lays the regions out differently and needs it
 *                zero-filled first.  Calls that overlap in time must use
 *                different workspaces.  NULL requests the size only:
 *                *workspace_bytes is set to the size required and nothing is
 *                launched.
 * workspace_bytes in: bytes available at workspace; out (size query): bytes
 *                required.  Must not be NULL.
 * stream         HIP stream to enqueue on (0 = null stream).
 *
 * Device data is not validated (that would need a synchronisation): logits
 * that are all -inf in a position, or NaN anywhere, give unspecified tokens
 * but every memory access stays in bounds.
 */
int spec_verify(const void* target_logits, const void* draft_logits,
                const int32_t* draft_tokens, const float* uniforms,
                const float* temperature, int B, int K, int V, int topk_draft,
                int dtype, int32_t* out_tokens, int32_t* num_accepted,
                void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * spec_verify_probe - spec_verify plus diagnostics, for parity tests.  Not
 * part of the serving API.
 *
 * probs_out  [B, K, 2] float32 device or NULL: (p_i(d_i), q_i(d_i)) for every
 *            position i < K of sampling rows (also after the first
 *            rejection); 0 for greedy rows.
 * mass_out   [B] float32 device or NULL: total weight S of the distribution
 *            the final token was drawn from (residual mass after a rejection,
 *            about 1 for the bonus); 0 for greedy rows.
 * Other arguments and return codes as spec_verify.
 */
int spec_verify_probe(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms,
                      const float* temperature, int B, int K, int V,
                      int topk_draft, int dtype, int32_t* out_tokens,
                      int32_t* num_accepted, void* workspace,
                      size_t* workspace_bytes, hipStream_t stream,
                      float* probs_out, float* mass_out);

/*
 * spec_verify_relaxed - spec_verify with a lossy relaxed acceptance rule in
 * place of u*q < p ("Acceptance Is Not Speed (arXiv:2610.23818): ...",
 * newsaint.id: section 1 describes verification that tolerates q > p within
 * a divergence budget, section 6 gives the budget's rule and a support guard,
 * section 7 recommends a strict support filter).  For each draft d_i of a
 * sampling row, in order:
 *   1. support guard: reject if d_i is outside [0, V), if its target rank
 *      1 + #{x : l_i(x) > l_i(d_i)} exceeds max_rank (max_rank = 0 disables
 *      the rank check), or if p_i(d_i) < min_prob;
 *   2. strict branch: accept if p_i(d_i) > 0 and q_i(d_i) <= p_i(d_i);
 *   3. otherwise accept iff u_i * q < gamma, gamma = min(p + sqrt(2 alpha p
 *      (1 - p)), 1) with p = p_i(d_i), q = q_i(d_i).
 * The first rejection ends the prefix as in spec_verify, and the correction
 * is drawn from the same residual norm(max(0, p_n - q_n)) (the pages leave
 * the correction under relaxed rules open; this is the plain reading).
 * Greedy rows (T <= 0) and the bonus draw are unchanged.  The output
 * distribution is no longer the target's: the rule is lossy by design.
 *
 * alpha     >= 0 divergence budget (0 with max_rank = 0 and min_prob = 0
 *           gives exactly spec_verify's decisions).
 * max_rank  >= 0 largest accepted target rank (0 = no rank check).  With a
 *           rank check the statistics pass also counts, per target position,
 *           the logits above l(d_i) (one compare per target logit).
 * min_prob  in [0, 1]: smallest accepted p_i(d_i).
 * probs_out, mass_out as spec_verify_probe (may be NULL).
 * Other arguments as spec_verify.  SV_ERR_ARG also for a negative or NaN
 * alpha, a negative max_rank or min_prob outside [0, 1].
 */
int spec_verify_relaxed(const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const float* uniforms,
                        const float* temperature, int B, int K, int V,
                        int topk_draft, int dtype, float alpha, int max_rank,
                        float min_prob, int32_t* out_tokens,
                        int32_t* num_accepted, void* workspace,
                        size_t* workspace_bytes, hipStream_t stream,
                        float* probs_out, float* mass_out);

/*
 * spec_verify_kl - spec_verify that also returns KL(p_i || q_i), in nats, for
 * every draft position of each sampling row: the distillation signal that
 * test-time speculation takes from the verification step (gist.science
 * summary of paper 2605.09329, section 2: KL between the target's and the
 * drafter's distributions over the verified positions, with position weights
 * applied by the caller).  The value is exact up to fp32 rounding:
 *   KL = E_p[l_t - l_q] / T - ln 2 (fl(M_t s) - fl(M_q s)) - ln Z_t + ln Z_q
 * with the chunk statistics of the verification pass (s = log2(e) / T).
 * The statistics pass pairs each draft position with its target position so
 * that both are read once; tokens and num_accepted equal spec_verify's up to
 * the rounding of p and q (their decisions use the same partial sums).
 *
 * kl_out  [B, K] float32 device: KL(p_i || q_i); NaN for greedy rows (no
 *         sampling distribution); +inf where the draft gives zero mass to a
 *         token the target can produce.  Required when K > 0.
 * A sparse draft (0 < topk_draft < V) is not supported (KL against a
 * truncated draft is +inf): SV_ERR_UNSUPPORTED.  Other arguments and return
 * codes as spec_verify.
 */
int spec_verify_kl(const void* target_logits, const void* draft_logits,
                   const int32_t* draft_tokens, const float* uniforms,
                   const float* temperature, int B, int K, int V,
                   int topk_draft, int dtype, int32_t* out_tokens,
                   int32_t* num_accepted, void* workspace,
                   size_t* workspace_bytes, hipStream_t stream, float* kl_out);

/*
 * spec_verify_early_exit - spec_verify that verifies the positions of a row
 * one after the other and stops reading its logits at the first rejection:
 * no later draft can be committed ("Speculative decoding: memverifikasi
 * token draft sebelum diterima", subsection "Penolakan memendekkan pekerjaan
 * speculative yang berguna").  A row that rejects at position n reads the
 * target and draft logits of positions 0..n only (plus the residual pass of
 * position n), instead of all 2K+1 positions; in exchange its positions are
 * verified in sequence rather than in parallel.  Tokens, counts, the
 * probabilities p_i(d_i), q_i(d_i) and the final mass equal spec_verify's
 * bit for bit.
 *
 * One kernel per call for a dense draft.  topk_draft as spec_verify: a
 * truncated draft's selection does not depend on any decision, so such a
 * call makes every position's selection before the walk (three kernels:
 * position 0's statistics and the drafts' candidate lists, the selections,
 * the walk); it reads all K drafts of a sampling row, and the targets up to
 * the first rejection.  A shape whose row statistics ((2K+1) C 16 + C 128
 * bytes, plus 16 topk_draft for a truncated draft) do not fit the walking
 * kernel's LDS is SV_ERR_UNSUPPORTED.  The workspace has its own size (query
 * with workspace == NULL) and must not be shared with the other entry
 * points: each call leaves it ready for the next call of the same shape (a
 * dense draft leaves it all zero); zero-fill it before a call of another
 * shape.
 * probs_out  [B, K, 2] float32 device or NULL: (p_i(d_i), q_i(d_i)) of every
 *            position the row tested, NaN past its first rejection (and for
 *            greedy rows).
 * mass_out   [B] float32 device or NULL: as spec_verify_probe.
 * Other arguments and return codes as spec_verify.
 */
int spec_verify_early_exit(const void* target_logits, const void* draft_logits,
                           const int32_t* draft_tokens, const float* uniforms,
                           const float* temperature, int B, int K, int V,
                           int topk_draft, int dtype, int32_t* out_tokens,
                           int32_t* num_accepted, void* workspace,
                           size_t* workspace_bytes, hipStream_t stream,
                           float* probs_out, float* mass_out);

/*
 * spec_verify_tree - verify B rows of draft trees against one target pass
 * (RheoSampling 2026, section 4, RheoVerification: sibling candidates are
 * tested one after the other; an accepted candidate is descended into; after
 * a rejection the next sibling is tested against the residual
 * norm(max(0, r - q~)); when every candidate is rejected the final token is
 * drawn from the last residual).
 *
 * A row's tree has N nodes; node 0 is the root (the committed prefix) and
 * every other node c is a candidate token tok[c] drawn, independently of its
 * siblings, from the drafter's distribution at its parent par[c] < c.
 * Children are tested in increasing node index.  With r_0 = p_v at node v,
 * the j-th tested child (0-based) is accepted when u[c] * q_v(d) < r_j(d),
 * where r_j = max(0, p_v - c_j q_v) / W_j, c_0 = 0, W_0 = 1,
 * c_{j+1} = c_j + W_j, W_j = sum_x max(0, p_v(x) - c_j q_v(x)).  A rejection
 * therefore costs one pass over node v's target and draft logits (for the
 * next W).  A leaf reached by acceptance emits a bonus token drawn from its
 * target p_leaf.  Greedy rows (T <= 0) descend into the first child whose
 * token equals the node's target argmax and emit the argmax where none does.
 * Every draw is the inverse CDF of spec_verify with uniform u[b][0].  A chain
 * (par[c] = c - 1) gives exactly spec_verify's result with K = N - 1,
 * draft_tokens[i] = tok[i+1] and uniforms (u[1..N-1], u[0]).
 *
 * target_logits  [B, N, V] device, dtype: the target's next-token logits at
 *                each node (after the path root..node).
 * draft_logits   [B, N, V] device, dtype: the drafter's logits at each node;
 *                read only for nodes with children (other rows may hold any
 *                values) and never for greedy rows.
 * node_tokens    [B, N] int32 device; entry 0 is not read.  A token outside
 *                [0, V) has p = q = 0 and is rejected.
 * parents        [B, N] int32 device; entry 0 is not read.  par[c] must be
 *                < c; a node whose parent is not an earlier node is never
 *                reached.
 * uniforms       [B, N] float32 device in [0, 1): u[c] tests node c, u[0]
 *                drives the final draw.
 * temperature    [B] float32 device; T <= 0 (or NaN) selects greedy.
 * B >= 1, N in [1, SV_MAX_NODES], V >= 1.
 * topk_draft     0 or >= V: dense drafts; otherwise every node's draft is cut
 *                to its topk_draft largest logits (at most SV_MAX_TOPK), as in
 *                spec_verify, and a third kernel selects each node's kept set.
 * out_tokens     [B, N] int32 device: the tokens of the accepted nodes in
 *                path order, then the final token, then -1.
 * out_nodes      [B, N] int32 device: the accepted node indices in path
 *                order, then -1.
 * num_accepted   [B] int32 device: accepted nodes (-1 if a wait for another
 *                work-group's results timed out, which a correct launch
 *                never does).
 * workspace, workspace_bytes, stream as spec_verify (the size depends on
 *                B, N, V and dtype).
 * probs_out      [B, N, 3] float32 device or NULL: (p_v(d), q_v(d), r_j(d))
 *                of every tested node, NaN for nodes not tested.
 * mass_out       [B] float32 device or NULL: total weight of the final
 *                draw's distribution (W for a residual, ~1 for a target), 0
 *                for greedy rows.
 * Every call enqueues two kernels (three with a sparse draft).
 * SV_ERR_UNSUPPORTED also when the row's chunk statistics (2 N C 16 bytes,
 * plus 12 topk_draft bytes) do not fit the walking kernel's LDS.
 */
int spec_verify_tree(const void* target_logits, const void* draft_logits,
                     const int32_t* node_tokens, const int32_t* parents,
                     const float* uniforms, const float* temperature, int B,
                     int N, int V, int topk_draft, int dtype,
                     int32_t* out_tokens, int32_t* out_nodes,
                     int32_t* num_accepted, void* workspace,
                     size_t* workspace_bytes, hipStream_t stream,
                     float* probs_out, float* mass_out);

/*
 * spec_verify_tree_timed - spec_verify_tree (without probes) that also times
 * its kernels: events[0] / events[1] take the start / end of the statistics
 * kernel's dispatch, events[2] / events[3] those of the walking kernel (a
 * sparse draft's selection kernel runs between them, untimed).
 * n_events must be 4.
 */
int spec_verify_tree_timed(const void* target_logits, const void* draft_logits,
                           const int32_t* node_tokens, const int32_t* parents,
                           const float* uniforms, const float* temperature,
                           int B, int N, int V, int topk_draft, int dtype,
                           int32_t* out_tokens, int32_t* out_nodes,
                           int32_t* num_accepted, void* workspace,
                           size_t* workspace_bytes, hipStream_t stream,
                           hipEvent_t* events, int n_events);

/*
 * spec_verify_timed - spec_verify that also times each of its kernels on the
 * caller's stream, for measurement.
 *
 * events     array of n_events events created by the caller (hipEventCreate).
 *            events[0] / events[1] take the start / end timestamps of the
 *            statistics kernel's dispatch, events[2] / events[3] those of the
 *            sparse-draft merge kernel (both recorded after the statistics
 *            kernel when there is none), events[4] / events[5] those of the
 *            finishing kernel (decision, residual mass and final draw).
 *            n_events must be 0 or 6.
 * Other arguments and return codes as spec_verify.
 */
int spec_verify_timed(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms,
                      const float* temperature, int B, int K, int V,
                      int topk_draft, int dtype, int32_t* out_tokens,
                      int32_t* num_accepted, void* workspace,
                      size_t* workspace_bytes, hipStream_t stream,
                      hipEvent_t* events, int n_events);

/*
 * spec_verify_noalloc - spec_verify for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, semantics and results as spec_verify
 * (bit for bit), without the workspace: the scratch is a static device array
 * of SV_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  Its device address is looked up once per device, on the
 * first call made with that device current.  Each call clears the part of
 * the scratch its shape uses with a small fill kernel on `stream` (no
 * memory set, so it can be captured) and then enqueues spec_verify's kernels.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).
 *
 * Every call on a GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (different streams, or graphs replayed concurrently) race and
 * must not be issued; calls serialised on one stream are fine.
 * Returns SV_ERR_SCRATCH, before enqueuing anything, when the shape's
 * workspace (spec_verify's size query) exceeds SV_SCRATCH_BYTES -- a dense
 * draft of 256 rows, K = 7, V = 201,088 needs about 1.7 MB; truncated drafts
 * need about 2 KB per (row, position, vocabulary chunk) more up to
 * topk_draft = 128 (8 bytes per candidate entry, max(256, topk_draft, about
 * 4.5 topk_draft / C + 24) entries per chunk).  SV_ERR_HIP if
 * the scratch's address cannot be obtained.  Other codes as spec_verify.
 */
int spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const float* uniforms,
                        const float* temperature, int B, int K, int V,
                        int topk_draft, int dtype, int32_t* out_tokens,
                        int32_t* num_accepted, hipStream_t stream);

/*
 * spec_verify_launches - how many kernels a spec_verify (or _probe, _relaxed,
 * _timed) call of this shape enqueues: 2 for a dense draft (statistics,
 * finishing), 3 with a truncated draft (statistics, selection, finishing);
 * spec_verify_noalloc enqueues one more (the fill of its scratch).  A
 * negative value is minus an sv_status for a shape spec_verify refuses.
 */
int spec_verify_launches(int B, int K, int V, int topk_draft, int dtype);

/*
 * spec_verify_plan - the vocabulary split the library would use for a shape:
 * *chunks vocabulary chunks per (row, position), each *chunk_len ids long
 * (the last one may be shorter).  For tests that need inputs spanning several
 * chunks and a ragged tail.  Returns SV_OK or SV_ERR_ARG / SV_ERR_UNSUPPORTED.
 */
int spec_verify_plan(int B, int K, int V, int topk_draft, int dtype,
                     int* chunks, int* chunk_len);

/* Static description of a status code (never NULL). */
const char* spec_verify_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
