/*
 * ra.h - C ABI of a blockwise ring-attention library for AMD MI355X (gfx950).
 *
 * One GPU's share of context-parallel ring attention: a local query shard is
 * swept over the key/value chunks of a sequence in ring order; each chunk step
 * yields a partial output and its log-sum-exp (LSE); partials are merged by
 * LSE rescaling; the backward recomputes every step against that step's own
 * K/V chunk.  Pages cited (titles shortened):
 *   [P1] diffusers issue "Ring attention backward uses stale iteration-0 KV
 *        from ctx.saved_tensors - silent gradient corruption when training
 *        with context parallelism"
 *   [P2] DeepSpeed PR "[bugfix] _DimZeroAllToAll silently fails to send grads
 *        under torch.compile"
 *   [P3] diffusers PR "Fix Flux Context Parallel Bug (Incoherent Image
 *        Generation)"
 *   [P4] DeepSpeed issue "[BUG] DistributedAttention produces numerically
 *        incorrect results vs its own SeqAllToAll-equivalent baseline when
 *        sequence length is not divisible by world size"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory: every pointer in a tensor descriptor is DEVICE memory owned by the
 *   caller; the library never allocates or frees device memory.  Host arrays
 *   (chunk tables, tensor arrays, size outputs) are read/written during the
 *   call only.  Scratch space is passed in as a caller-owned workspace (except
 *   for ra_ring_fwd_noalloc, which uses a device array of the library itself).
 * Streams: `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue
 *   work and return without synchronising; pointers must stay valid until the
 *   enqueued work completes.  The library keeps no global state beyond a
 *   thread-local error string and, for ra_ring_fwd_noalloc, that device array
 *   and its per-device address (looked up once, under a lock), so every entry
 *   point is thread-safe; concurrent ra_ring_fwd_noalloc calls on one GPU
 *   share its array (see there).
 * Layout: an ra_tensor is a logical [B, S, H, D] tensor with element strides
 *   sB, sS, sH and D contiguous (stride 1).  Batch-first [B,S,H,D] ([P1]
 *   "Reproduction") and sequence-first [S,B,H,D] ([P4] "Testcase") are the same
 *   logical tensor with other strides; a sequence chunk is a pointer offset
 *   plus a length.  No entry point copies or permutes to change layout.
 * Dtypes: inputs q, k, v, dout are all bf16 or all fp32.  Accumulators
 *   (partial/running outputs, dq/dk/dv accumulators) and LSE/delta are fp32.
 *   bf16 conversions round to nearest even.
 * LSE: fp32 [B, H_q, S_q] (ra_lse), natural logarithm, S contiguous.
 * GQA: H_kv must divide H_q; query head h uses key/value head h / (H_q/H_kv).
 * Scale: the softmax scale is an argument; the Python binding passes
 *   1/sqrt(D) (the SDPA default of [P1] "Reproduction") when none is given.
 *   It must be finite and >= 2^-100 (RA_E_ARG otherwise): the bf16 dK/dV
 *   kernel starts its score accumulator at -lse / scale.
 *   There is no dropout, causal mode or general attention mask ([P4]
 *   "Testcase" calls attention with None, 0.0, False); none is offered, so
 *   none can be silently ignored.  The one mask offered is a key-validity
 *   (key-padding) mask, through the *_masked entry points below.
 * Errors: each call validates all arguments on the host BEFORE any launch and
 *   returns a status; on failure nothing has been enqueued and ra_last_error()
 *   describes the problem.  Anything the library cannot compute exactly is
 *   refused (silent wrong results are the failure mode all four pages report).
 *   A launch failure reported by HIP returns RA_E_HIP.
 * Supported: D in {64, 128}; 16-byte aligned data pointers and strides that
 *   are multiples of 16 bytes; B, H >= 1; any S >= 0 (tails are masked, never
 *   padded: [P3] thread, padding changes the result).
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RA_OK = 0,
    RA_E_ARG = 1,          /* null pointer, negative size, bad flag */
    RA_E_SHAPE = 2,        /* shapes inconsistent (incl. H_q % H_kv != 0) */
    RA_E_DTYPE = 3,        /* dtype combination not supported */
    RA_E_ALIGN = 4,        /* pointer or stride not 16-byte aligned */
    RA_E_UNSUPPORTED = 5,  /* valid request outside what is built (e.g. D=96) */
    RA_E_WORKSPACE = 6,    /* workspace missing or too small */
    RA_E_HIP = 7           /* HIP reported an error at launch */
} ra_status;

typedef enum { RA_BF16 = 1, RA_F32 = 2 } ra_dtype;

/* Logical [B, S, H, D] tensor; element (b,s,h,d) lives at
 * data + (b*sB + s*sS + h*sH + d) * sizeof(dtype). */
typedef struct {
    void*   data;
    int32_t dtype;      /* ra_dtype */
    int32_t B, S, H, D;
    int64_t sB, sS, sH; /* element strides */
} ra_tensor;

/* fp32 [B, H, S] per-row statistic (LSE or delta); element (b,h,s) at
 * data[b*sB + h*sH + s]. */
typedef struct {
    float*  data;
    int32_t B, H, S;
    int64_t sB, sH;
} ra_lse;

/* Chunk table of the key/value sequence.  Chunk c covers rows
 * [start[c], start[c] + len[c]) of k and v; the chunks must tile [0, S_k)
 * exactly (empty chunks allowed).  order[i] is the chunk swept at step i and
 * must be a permutation of 0..n-1.  ([P1] "Root cause": step 0 of a rank's
 * ring is its local chunk; ra_ring_order builds that order.) */
typedef struct {
    int32_t        n;
    const int32_t* start;
    const int32_t* len;
    const int32_t* order;
} ra_chunks;

/* Key-validity mask of a key sequence (key padding): key s of batch b takes part
 * in attention iff data[b*sB + s] != 0.  uint8 in device memory, S contiguous.
 * [P3] (comments on padding to a length divisible by the world size): padded
 * tokens change the result because they are attended, and masking them is the
 * way to keep padded inputs exact.  Masked keys leave every softmax of their
 * batch; a query row of a batch with no valid key in the swept keys gets
 * out = 0, lse = -inf and zero gradients; masked keys get dK = dV = 0.
 * Where a *_masked entry point takes k as a chunk, the mask covers that chunk
 * (S = its S_k); for the ring sweeps it covers the whole key sequence and is
 * sliced with the chunks.  A NULL mask pointer means no mask. */
typedef struct {
    const uint8_t* data;
    int32_t B, S;
    int64_t sB;
} ra_kmask;

/* ---------------------------------------------------------------- chunk steps */

/* One forward chunk step ([P1] "Root cause": per ring iteration the attention
 * op returns out and lse).  q: [B,S_q,H_q,D]; k, v: the chunk [B,S_k,H_kv,D]
 * (S_k may be 0).  out: fp32 [B,S_q,H_q,D]; lse: [B,H_q,S_q].
 * merge = 0: write the chunk's partial result (normalised output, LSE); an
 *            empty chunk writes out = 0, lse = -inf (the merge identity).
 * merge = 1: LSE-merge the chunk's partial into the running (out, lse)
 *            in place ([P1] "How it surfaces per backend": ring needs LSE
 *            for partial-result merging); an empty chunk changes nothing. */
ra_status ra_fwd_chunk(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                       float scale, ra_tensor* out, ra_lse* lse, int32_t merge,
                       void* stream);

/* Merge two partial results over disjoint key sets, in place into (out_acc,
 * lse_acc): lse = log(e^lse_acc + e^lse_part), out = e^(lse_acc-lse) out_acc
 * + e^(lse_part-lse) out_part.  All fp32, same shapes.  A side at -inf is the
 * identity; both at -inf give (0, -inf).  ([P1] "How it surfaces per backend".) */
ra_status ra_merge_lse(ra_tensor* out_acc, ra_lse* lse_acc,
                       const ra_tensor* out_part, const ra_lse* lse_part, void* stream);

/* delta[b,h,s] = sum_d dout[b,s,h,d] * out[b,s,h,d] with the FINAL merged
 * output (fp32 or bf16 out; dout bf16 or fp32).  Used by the backward. */
ra_status ra_bwd_delta(const ra_tensor* out, const ra_tensor* dout, ra_lse* delta, void* stream);

/* One backward chunk step against THIS step's own K/V chunk ([P1] "Root
 * cause" and "Expected behavior": the backward must see the same rotated chunk
 * as the forward did, never the chunk saved at step 0).  lse and delta are the
 * final (merged) statistics of the full sweep.
 *   dq_acc: fp32 [B,S_q,H_q,D], accumulated (+=) - dQ is local to the rank.
 *   dk_acc, dv_acc: fp32 [B,S_k,H_kv,D] of this chunk; accumulate = 0
 *   overwrites them, 1 adds to them.  GQA: a key/value head receives the sum
 *   over the query heads of its group. */
ra_status ra_bwd_chunk(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                       const ra_tensor* dout, const ra_lse* lse, const ra_lse* delta,
                       float scale, ra_tensor* dq_acc, ra_tensor* dk_acc, ra_tensor* dv_acc,
                       int32_t accumulate, void* stream);

/* The two halves of ra_bwd_chunk, for callers that schedule them separately (in a
 * ring, a step's dK/dV leave the rank while its dQ contribution stays local).
 * Same arguments and rules as ra_bwd_chunk; ra_bwd_chunk_dkdv touches only dk_acc
 * and dv_acc (accumulate = 0 overwrites, 1 adds), ra_bwd_chunk_dq only adds to
 * dq_acc. */
ra_status ra_bwd_chunk_dkdv(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                            const ra_tensor* dout, const ra_lse* lse, const ra_lse* delta,
                            float scale, ra_tensor* dk_acc, ra_tensor* dv_acc,
                            int32_t accumulate, void* stream);
ra_status ra_bwd_chunk_dq(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                          const ra_tensor* dout, const ra_lse* lse, const ra_lse* delta,
                          float scale, ra_tensor* dq_acc, void* stream);

/* The chunk steps with a key mask (kmask may be NULL: same as the entry points
 * above).  kmask covers the chunk k: B = q.B, S = k.S. */
ra_status ra_fwd_chunk_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                              const ra_kmask* kmask, float scale, ra_tensor* out, ra_lse* lse,
                              int32_t merge, void* stream);
ra_status ra_bwd_chunk_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                              const ra_tensor* dout, const ra_lse* lse, const ra_lse* delta,
                              const ra_kmask* kmask, float scale, ra_tensor* dq_acc,
                              ra_tensor* dk_acc, ra_tensor* dv_acc, int32_t accumulate, void* stream);
ra_status ra_bwd_chunk_dkdv_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                                   const ra_tensor* dout, const ra_lse* lse, const ra_lse* delta,
                                   const ra_kmask* kmask, float scale, ra_tensor* dk_acc,
                                   ra_tensor* dv_acc, int32_t accumulate, void* stream);
ra_status ra_bwd_chunk_dq_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                                 const ra_tensor* dout, const ra_lse* lse, const ra_lse* delta,
                                 const ra_kmask* kmask, float scale, ra_tensor* dq_acc, void* stream);

/* The bf16 chunk step by the stored-dS route (what ra_ring_bwd runs for bf16
 * inputs; the same step as ra_bwd_chunk, [P1] "Root cause" and "Expected
 * behavior": each backward step against its own chunk, dQ local, dK/dV of the
 * chunk): ra_bwd_chunk_dkdv_ds is ra_bwd_chunk_dkdv_masked that also writes
 * the step's dS = P (dP - delta) (bf16; zero for masked keys) to the device
 * buffer ds; ra_bwd_chunk_dq_ds then adds scale dS K to dq_acc (fp32) from that
 * buffer, with the same q (rows), k (chunk) and scale, without forming S and dP
 * again.  ds must hold ra_bwd_ds_bytes(q, k) bytes (256-byte aligned); its
 * layout is private to these two calls.  dk_acc/dv_acc may also be bf16
 * (shape of k) with accumulate = 0: the step's dK/dV are then final and
 * written there in bf16 (what ra_ring_bwd does when each chunk is one step;
 * with S_q = 0 that is refused, RA_E_UNSUPPORTED, as nothing would write
 * them).  bf16 inputs only (RA_E_DTYPE otherwise); ds too small or NULL:
 * RA_E_WORKSPACE.  The result equals ra_bwd_chunk's up
 * to rounding (P reaches dS through fp16 here). */
size_t ra_bwd_ds_bytes(const ra_tensor* q, const ra_tensor* k);
ra_status ra_bwd_chunk_dkdv_ds(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                               const ra_tensor* dout, const ra_lse* lse, const ra_lse* delta,
                               const ra_kmask* kmask, float scale, ra_tensor* dk_acc,
                               ra_tensor* dv_acc, int32_t accumulate, void* ds, size_t ds_bytes,
                               void* stream);
ra_status ra_bwd_chunk_dq_ds(const ra_tensor* q, const ra_tensor* k, const void* ds,
                             size_t ds_bytes, float scale, ra_tensor* dq_acc, void* stream);

/* ---------------------------------------------------------------- ring sweeps */

/* Forward sweep of the local query shard over every chunk in chunks->order:
 * step 0 writes the partial, later steps merge in the fused epilogue, then the
 * result is written to out (bf16 or fp32) and lse.  k, v hold the whole key
 * sequence [B,S_k,H_kv,D]; chunks tile it.  ws: device workspace of at least
 * ra_ring_fwd_workspace_bytes(q, out) bytes (fp32 running output when out is
 * bf16; 0 bytes needed when out is fp32).  With bf16 inputs and a bf16 out, the
 * last non-empty step writes the merged output to out directly, rounded to
 * nearest even: the same values as rounding the fp32 running output. */
ra_status ra_ring_fwd(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                      const ra_chunks* chunks, float scale, ra_tensor* out, ra_lse* lse,
                      void* ws, size_t ws_bytes, void* stream);

/* Backward sweep: delta from (out, dout), then one chunk step per chunk in
 * the same order as the forward, each against its own chunk; dq, dk, dv
 * (bf16 or fp32, shapes of q, k, v) are written.  ws: a device workspace of
 * ws_bytes bytes (256-byte aligned), at least
 * ra_ring_bwd_workspace_min_bytes(q, k, dq, dk, dv) (RA_E_WORKSPACE below
 * that); ra_ring_bwd_workspace_bytes gives the size that runs fastest.  With
 * bf16 inputs a chunk step computes the same quantities as ra_bwd_chunk by
 * another route: the dK/dV kernel stores dS = P (dP - delta) in bf16 to the
 * workspace and a second kernel forms dQ += scale dS K from it, instead of
 * recomputing S and dP.  The sweep plans from the room ws_bytes leaves: query
 * rows go in slices (multiples of 64) when the dS of a whole chunk does not fit,
 * and a chunk whose slices would be too thin to fill the GPU takes the
 * recompute route (ra_bwd_chunk's kernels).  When the dS of every chunk does not
 * fit at once but that of every chunk (at most 8) for a slice of 4096 or more
 * query rows does, the sweep runs slice by slice instead: each slice runs the
 * chunk steps of every chunk in sweep order, then one dQ pass over all of them
 * that writes the slice's dq rows.  Any plan gives the same result up to
 * rounding.  fp32 accumulators for bf16 gradients are carved only where the
 * plan needs them.  Results agree with ra_bwd_chunk up to rounding, not bit for
 * bit. */
ra_status ra_ring_bwd(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                      const ra_tensor* out, const ra_tensor* dout, const ra_lse* lse,
                      const ra_chunks* chunks, float scale,
                      ra_tensor* dq, ra_tensor* dk, ra_tensor* dv,
                      void* ws, size_t ws_bytes, void* stream);

/* The ring sweeps with a key mask over the whole key sequence (B = q.B,
 * S = k.S; sliced with the chunks).  kmask may be NULL.  Workspaces as above. */
ra_status ra_ring_fwd_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                             const ra_kmask* kmask, const ra_chunks* chunks, float scale,
                             ra_tensor* out, ra_lse* lse, void* ws, size_t ws_bytes, void* stream);
ra_status ra_ring_bwd_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                             const ra_tensor* out, const ra_tensor* dout, const ra_lse* lse,
                             const ra_kmask* kmask, const ra_chunks* chunks, float scale,
                             ra_tensor* dq, ra_tensor* dk, ra_tensor* dv,
                             void* ws, size_t ws_bytes, void* stream);

/* ra_ring_fwd_masked without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, validation, results and
 * errors as ra_ring_fwd_masked (kmask may be NULL).  It allocates and frees
 * nothing: the fp32 running output of a bf16 sweep lives in a device array of
 * the library (64 MiB per GPU, held until the process ends), so a sweep whose
 * ra_ring_fwd_workspace_bytes(q, out) exceeds 64 MiB (more than 16 Mi elements
 * of q) is refused with RA_E_WORKSPACE before anything is enqueued.  The first
 * call on a device looks the array's address up (a runtime query, no
 * allocation; callers that capture graphs make one call before capturing).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (other streams, other threads) race and must be serialised by the
 * caller; calls in one stream are ordered as usual. */
ra_status ra_ring_fwd_noalloc(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v,
                              const ra_kmask* kmask, const ra_chunks* chunks, float scale,
                              ra_tensor* out, ra_lse* lse, void* stream);

/* Workspace sizes.  ra_ring_fwd_workspace_bytes: what ra_ring_fwd needs.
 * ra_ring_bwd_workspace_min_bytes: ra_ring_bwd accepts any workspace of at least
 * this size with any chunk table: delta plus an fp32 accumulator for every bf16
 * gradient (every chunk may then take the recompute route).  With a given chunk
 * table a plan may need less (e.g. chunks small enough to keep the stored-dS
 * route with no dK/dV accumulators); ra_ring_bwd refuses a workspace only when
 * the plan it allows needs more than ws_bytes.  ra_ring_bwd_workspace_bytes: the
 * size at which ra_ring_bwd runs fastest: delta, the fp32 accumulators its plan
 * needs and a dS region of min(8 GiB, dS of every query row against the whole
 * key sequence plus 7 key tiles of 128, the rounding to whole tiles that a table
 * of up to 8 chunks adds), and never less than the minimum.  dq/dk/dv give the
 * gradient dtypes (NULL: the dtype of q/k/v). */
size_t ra_ring_fwd_workspace_bytes(const ra_tensor* q, const ra_tensor* out);
size_t ra_ring_bwd_workspace_bytes(const ra_tensor* q, const ra_tensor* k,
                                   const ra_tensor* dq, const ra_tensor* dk, const ra_tensor* dv);
size_t ra_ring_bwd_workspace_min_bytes(const ra_tensor* q, const ra_tensor* k,
                                       const ra_tensor* dq, const ra_tensor* dk, const ra_tensor* dv);

/* The plan ra_ring_bwd_masked would run for these arguments with a workspace of
 * ws_bytes bytes, computed on the host (no launch, no device access): q and k
 * validated as ra_ring_bwd validates them (k standing in for v), the gradients'
 * dtypes (NULL: the dtype of q/k) and the chunk table; then *slice_rows = the
 * query rows per slice when the sweep runs slice
 * by slice (0: chunk by chunk); rows[i] (chunks->n entries, i-th chunk of the
 * sweep order) = the query rows per dK/dV launch of that chunk on the stored-dS
 * route, 0 on the recompute route, -1 for an empty chunk (or no query rows);
 * *accs = bit 0, 1, 2 set when an fp32 accumulator for dq, dk, dv is carved from
 * the workspace.  RA_E_WORKSPACE when ws_bytes is below what that plan needs.
 * Any output pointer may be NULL. */
ra_status ra_ring_bwd_plan(const ra_tensor* q, const ra_tensor* k, const ra_tensor* dq,
                           const ra_tensor* dk, const ra_tensor* dv, const ra_chunks* chunks,
                           size_t ws_bytes, int32_t* slice_rows, int32_t* rows, uint32_t* accs);

/* ---------------------------------------------------------------- exchange */

/* Ulysses-style sequence<->head exchange of R simulated ranks, done in-device
 * as a bit-exact block permutation ([P4] "Testcase": all-to-all scattering
 * heads and gathering sequence, and its inverse; [P2] "Testing": slot i of a
 * rank's output is the slot that rank owns in rank i's input).
 * dir = 0 (seq->head): in[i] is rank i's sequence shard [B, s_i, H, D];
 *   out[r] is rank r's head group [B, S, h_r, D], S = sum s_i, sum h_r = H,
 *   out[r][b, off_i + t, c, :] = in[i][b, t, hoff_r + c, :].
 * dir = 1 (head->seq): the inverse (in[r] are head groups, out[i] shards).
 * s_i and h_r are read from the descriptors' S and H fields, so uneven splits
 * (e.g. 334/333/333 rows, 3/3/2 heads) need no padding.  Both dtypes; in and
 * out must have the same dtype; 1 <= R <= 16; in and out must not overlap. */
ra_status ra_seq_head_permute(const ra_tensor* in, int32_t n_in, ra_tensor* out, int32_t n_out,
                              int32_t dir, void* stream);

/* ---------------------------------------------------------------- host helpers */

/* Sizes of `parts` consecutive pieces of n, the first n % parts one larger
 * (1000/3 -> 334,333,333).  sizes must hold `parts` entries. */
ra_status ra_split_sizes(int32_t n, int32_t parts, int32_t* sizes);

/* Ring order of `rank` in a ring of R: step i sweeps chunk (rank - i) mod R,
 * so step 0 is the local chunk ([P1] "Root cause").  order holds R entries. */
ra_status ra_ring_order(int32_t R, int32_t rank, int32_t* order);

const char* ra_status_string(ra_status s);
/* Detail of the last failure on the calling thread (empty if none).  For
 * H_q % H_kv != 0 it contains the message quoted in [P1] "How it surfaces per
 * backend": "Number of heads in key/value must divide number of heads in query". */
const char* ra_last_error(void);
/* Library version string. */
const char* ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
