/*
 * hyattn -- per-layer attention step of a hybrid full/linear-attention model
 * on AMD Instinct MI355X (gfx950). C ABI.
 *
 * Pages cited (by title and section):
 *   P2 = "推理框架适配Hybrid Model：KV Cache管理与算子调度实战"
 *   P1 = "Hybrid Model推理适配：vLLM与SGLang的工程实践指南"
 *
 * What the library computes (P2 §2.1, §2.3):
 *   - linear layers keep, per request and head, a D x D fp32 state S. Each new
 *     token adds k (x) v to S (S[i][j] += k[i] * v[j]) and the layer outputs
 *     o = q . S (o[j] = sum_i q[i] S[i][j]) using the state that already holds
 *     that token. Chunked prefill gives the same result chunk by chunk
 *     (P2 §2.4); decode updates S in place.
 *   - full layers keep K and V in a pool of 16-token blocks reached through a
 *     per-request block table; attention is softmax(scale * q . k) . v over
 *     the request's cached tokens (causal inside a prefill chunk).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates or frees device memory. Host pointers are marked "host".
 *   - Element types: q/k/v/o and KV pools are fp32 or bf16 (hyattn_dtype);
 *     linear states are always fp32. bf16 outputs are rounded to nearest-even.
 *   - Layouts are row-major, innermost dimension last:
 *       packed tokens  [N_tok][H][D]         (token-major)
 *       KV pool        [n_blocks][H_kv][16][D]
 *       block tables   int32 [B][max_blocks_per_seq], -1 = unused entry
 *       state pool     fp32 [n_linear_layers][n_slots][H][D][D]
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call that
 *     launches work is asynchronous on that stream and never synchronizes,
 *     except in checked mode (environment HYATTN_CHECK=1), where calls copy
 *     index arrays to the host and validate their contents first.
 *   - Errors: every call validates its arguments before launching anything;
 *     a call that fails has no side effects. The message of the last failure
 *     on the calling thread is returned by hyattn_last_error().
 *   - Supported head dims: D = 64 and D = 128.
 */
#ifndef HYATTN_H
#define HYATTN_H

#include <stddef.h>
#include <stdint.h>

/* Tokens per block of the paged KV cache (P2 §2.1: fixed 16-token pages). */
#define HYATTN_BLOCK_TOKENS 16

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HYATTN_OK = 0,
  HYATTN_ERR_INVALID_ARG = 1,       /* null pointer, bad size, bad index content */
  HYATTN_ERR_OUT_OF_SLOTS = 2,      /* state pool exhausted (P2 §4.2, second OOM kind) */
  HYATTN_ERR_BAD_SLOT = 3,          /* slot id out of range, not allocated, or never zeroed */
  HYATTN_ERR_UNSUPPORTED_LAYER = 4, /* a layer type outside hyattn_layer_type (P1 §4.3) */
  HYATTN_ERR_UNSUPPORTED = 5,       /* D, dtype or chunk size without a kernel */
  HYATTN_ERR_HIP = 6                /* a HIP runtime call or launch failed */
} hyattn_status;

typedef enum { HYATTN_F32 = 0, HYATTN_BF16 = 1 } hyattn_dtype;

/* Layer types of the model config (P2 §2.2 "layer_types"). */
typedef enum { HYATTN_LAYER_LINEAR = 0, HYATTN_LAYER_FULL = 1 } hyattn_layer_type;

typedef struct hyattn_state_pool hyattn_state_pool; /* opaque host-side handle */

/* Thread-local text of the last error ("" after success). Never NULL. */
const char* hyattn_last_error(void);

/* ABI version of this header (bumped on incompatible changes). */
int hyattn_abi_version(void);

/* ---------------------------------------------------------------------------
 * State pool (P2 §1.3, §2.2, §2.3): a fixed-size fp32 state per request and
 * linear layer, separate from the paged KV pool, allocated and zeroed when a
 * request starts and released when it ends. Its size does not depend on the
 * sequence length.
 */

/* Bytes of a pool: n_linear_layers * n_slots * H * D * D * 4. 0 on overflow. */
size_t hyattn_state_pool_bytes(int n_linear_layers, int n_slots, int H, int D);

/* Wrap a caller-owned device buffer of at least hyattn_state_pool_bytes()
 * bytes (16-byte aligned). The handle owns only host bookkeeping; all slots
 * start free. D is 64 or 128 and H * D below 2^23 (HYATTN_ERR_UNSUPPORTED
 * otherwise). */
hyattn_status hyattn_state_pool_create(void* dev_buf, size_t bytes, int n_linear_layers,
                                       int n_slots, int H, int D, hyattn_state_pool** out);

/* Release the handle (not the device buffer). NULL is accepted. */
hyattn_status hyattn_state_pool_destroy(hyattn_state_pool* pool);

/* Host, synchronous, thread-safe. Reserve n slots: the n lowest free ids in
 * ascending order are written to slots_out (host). All-or-nothing: fails with
 * HYATTN_ERR_OUT_OF_SLOTS and changes nothing when fewer than n are free. */
hyattn_status hyattn_state_pool_alloc(hyattn_state_pool* pool, int n, int32_t* slots_out);

/* Zero the state of the given slots in every linear layer (request start).
 * slots_dev: device int32[n]; asynchronous on `stream`. In checked mode the
 * slots must be allocated. Marks the slots as zeroed for checked mode. */
hyattn_status hyattn_state_pool_zero(hyattn_state_pool* pool, const int32_t* slots_dev, int n,
                                     void* stream);

/* Host, synchronous. Return slots (host int32[n]) to the pool. Fails with
 * HYATTN_ERR_BAD_SLOT, changing nothing, if an id is out of range, not
 * allocated, or repeated. */
hyattn_status hyattn_state_pool_free(hyattn_state_pool* pool, const int32_t* slots, int n);

/* Number of slots currently allocated (the pool's memory-usage verb), or -1. */
int hyattn_state_pool_in_use(const hyattn_state_pool* pool);

/* Device address of the state S[layer][slot][0][0][0], or NULL if out of range. */
void* hyattn_state_pool_state_ptr(const hyattn_state_pool* pool, int linear_layer, int slot);

/* ---------------------------------------------------------------------------
 * Linear layers (P2 §2.1 recurrence; P2 §2.3 contract (Q, K, V, previous
 * state) -> (output, new state); P2 §2.4 chunked prefill).
 */

/* Chunked prefill of n_req packed requests on linear layer `linear_layer`.
 *   q, k, v, o   [N_tok][H][D], dtype; request r owns tokens
 *                cu_seqlens[r] .. cu_seqlens[r+1]-1 (device int32[n_req+1],
 *                non-decreasing, cu_seqlens[0] = 0).
 *   slots_dev    device int32[n_req]: the state slot of each request; the
 *                state is read as the prior state and overwritten in place.
 *   chunk_size   tokens per chunk: a multiple of 16 in [16, 256] (bf16);
 *                in [1, 128] for fp32 I/O. For each chunk c (the last may be
 *                shorter): O_c = Q_c S + tril(Q_c K_c^T) V_c, then
 *                S <- S + K_c^T V_c. Every chunking gives the same sums
 *                (P2 §2.4), so results differ between chunk sizes by
 *                rounding only; the bf16 kernel always works in 32-token
 *                blocks (streamed through LDS), the fp32 kernel in chunks of
 *                chunk_size.
 * Requests with zero tokens are left untouched. */
hyattn_status hyattn_linear_prefill_chunked(hyattn_state_pool* pool, int linear_layer,
                                            const void* q, const void* k, const void* v, void* o,
                                            const int32_t* cu_seqlens_dev,
                                            const int32_t* slots_dev, int n_req, int chunk_size,
                                            hyattn_dtype dtype, void* stream);

/* One decode step for B requests: per request r and head h,
 * S <- S + k (x) v, then o = q . S.  q, k, v, o: [B][H][D], dtype. */
hyattn_status hyattn_linear_decode(hyattn_state_pool* pool, int linear_layer, const void* q,
                                   const void* k, const void* v, void* o,
                                   const int32_t* slots_dev, int B, hyattn_dtype dtype,
                                   void* stream);

/* Gated (decayed) linear layer: the same calls with a per-token forget factor,
 * the nearest relative of the linear layer among the state-update variants
 * the pages point to (P2 §1.3: Mamba- and RWKV-style layers; P1 §2.1: a
 * state carried as h_t = f(h_{t-1}, x_t)). Token t of head h brings
 * g = log_gamma[t][h] (device fp32 [N_tok][H]; decode: [B][H]), finite and
 * <= 0 (checked in HYATTN_CHECK mode), and
 *     S <- exp(g) S + k (x) v,   o = q . S.
 * Chunked form, per chunk with L_a = g_0 + ... + g_a over the chunk:
 *     O_c = diag(exp(L)) Q_c S + (tril(Q_c K_c^T) * exp(L_a - L_b)) V_c,
 *     S  <- exp(L_last) S + K_c^T diag(exp(L_last - L_b)) V_c.
 * log_gamma = 0 everywhere gives the plain layer's results. Other arguments,
 * limits and errors as for the plain calls; log_gamma must not be NULL. */
hyattn_status hyattn_linear_prefill_chunked_gated(hyattn_state_pool* pool, int linear_layer,
                                                  const void* q, const void* k, const void* v,
                                                  const float* log_gamma, void* o,
                                                  const int32_t* cu_seqlens_dev,
                                                  const int32_t* slots_dev, int n_req,
                                                  int chunk_size, hyattn_dtype dtype,
                                                  void* stream);
hyattn_status hyattn_linear_decode_gated(hyattn_state_pool* pool, int linear_layer, const void* q,
                                         const void* k, const void* v, const float* log_gamma,
                                         void* o, const int32_t* slots_dev, int B,
                                         hyattn_dtype dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Full layers: paged KV cache of 16-token blocks (P2 §2.1 page table, P2 §2.3
 * PagedAttention decode, P1 §2.1 16 tokens per page).
 *
 * Logical token p of request r is stored in physical block
 * block_tables[r][p / 16] at offset p % 16, i.e. element
 * ((block * H_kv + g) * 16 + p % 16) * D of a pool, for KV head g.
 * context_lens (device int32[B]) count every cached token INCLUDING the new
 * ones of this step. Query head h reads KV head h / (H_q / H_kv).
 */

/* Write new tokens into the pools. k_new, v_new: [N_new][H_kv][D]; request r
 * owns rows cu_q_lens[r] .. cu_q_lens[r+1]-1 (device int32[B+1]); its i-th
 * new token goes to logical position context_lens[r] - q_len_r + i.
 * max_q_len (host) bounds the q lengths. */
hyattn_status hyattn_paged_append(const void* k_new, const void* v_new, void* k_pool,
                                  void* v_pool, int64_t n_blocks, const int32_t* block_tables_dev,
                                  int max_blocks_per_seq, const int32_t* context_lens_dev,
                                  const int32_t* cu_q_lens_dev, int B, int max_q_len, int H_kv,
                                  int D, hyattn_dtype dtype, void* stream);

/* Workspace (device bytes) needed by hyattn_paged_decode for B requests whose
 * contexts are at most max_context tokens. */
size_t hyattn_paged_decode_workspace_bytes(int B, int H_q, int D, int max_context);

/* Decode attention: one query per request (the token at position
 * context_lens[r] - 1, already appended). q, o: [B][H_q][D], dtype.
 * o = softmax(scale * q K_r^T) V_r over the context_lens[r] cached tokens;
 * context_lens[r] == 0 gives o = 0. max_context (host) bounds context_lens.
 * workspace: device buffer of hyattn_paged_decode_workspace_bytes() bytes. */
hyattn_status hyattn_paged_decode(const void* q, void* o, const void* k_pool, const void* v_pool,
                                  int64_t n_blocks, const int32_t* block_tables_dev,
                                  int max_blocks_per_seq, const int32_t* context_lens_dev,
                                  int max_context, int B, int H_q, int H_kv, int D, float scale,
                                  void* workspace, size_t workspace_bytes, hyattn_dtype dtype,
                                  void* stream);

/* Decode attention exactly as hyattn_paged_decode (same arguments, same
 * kernels, same results bit for bit), for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. It takes no workspace: its partition partials and scan live
 * in a file-scope device array of HYATTN_NOALLOC_SCRATCH_BYTES per GPU, held
 * until the process ends, whose address is looked up on the first call on each
 * device. It calls no hipMalloc, hipFree or allocating routine. A bf16 call
 * that needs more scratch than that (hyattn_paged_decode_workspace_bytes sizes
 * the worst case; at most B * H_q * 64 * (D + 2) * 4 bytes plus the scan) fails
 * with HYATTN_ERR_INVALID_ARG before launching. Every call on a GPU shares its
 * array, so calls that overlap on one GPU (other streams, other threads) race;
 * nothing in the array needs to start at zero (each call writes what it reads).
 * fp32 I/O uses no scratch. */
#define HYATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hyattn_status hyattn_paged_decode_noalloc(const void* q, void* o, const void* k_pool,
                                          const void* v_pool, int64_t n_blocks,
                                          const int32_t* block_tables_dev, int max_blocks_per_seq,
                                          const int32_t* context_lens_dev, int max_context, int B,
                                          int H_q, int H_kv, int D, float scale,
                                          hyattn_dtype dtype, void* stream);

/* Causal prefill attention over paged KV (FlashAttention-style, P2 §2.3): the
 * i-th query of request r (row cu_q_lens[r] + i of q/o, [N_q][H_q][D]) sits at
 * position context_lens[r] - q_len_r + i and attends to keys 0 .. that
 * position, all read through the block table (earlier chunks included). */
hyattn_status hyattn_paged_prefill(const void* q, void* o, const void* k_pool,
                                   const void* v_pool, int64_t n_blocks,
                                   const int32_t* block_tables_dev, int max_blocks_per_seq,
                                   const int32_t* context_lens_dev, const int32_t* cu_q_lens_dev,
                                   int max_q_len, int B, int H_q, int H_kv, int D, float scale,
                                   hyattn_dtype dtype, void* stream);

/* ---------------------------------------------------------------------------
 * One attention step over all layers of a hybrid model (P2 §2.2 layer-type
 * registration and per-forward metadata; P1 §3.2 per-layer dispatch plan).
 */
typedef struct {
  const void* q; /* linear: [N][H][D];  full: [N][H][D]            */
  const void* k; /* linear: [N][H][D];  full: new keys [N][H_kv][D]   */
  const void* v; /* linear: [N][H][D];  full: new values [N][H_kv][D] */
  void* o;       /* [N][H][D] */
  void* k_pool;  /* full layers: [n_blocks][H_kv][16][D]; linear: unused */
  void* v_pool;
  const float* log_gamma; /* linear layers: NULL, or the gated variant's log forget
                             factors fp32 [N][H] (prefill rows, then decode rows);
                             full layers: must be NULL */
} hyattn_layer_io;

typedef struct {
  int n_prefill;                /* requests bringing a prompt chunk (rows first)  */
  int n_decode;                 /* requests bringing one token (rows after those) */
  const int32_t* cu_seqlens;    /* device [n_prefill+1], prefill token offsets    */
  int n_prefill_tokens;         /* host: cu_seqlens[n_prefill] (decode rows start here) */
  int max_prefill_len;          /* host bound on prefill chunk lengths            */
  const int32_t* prefill_slots; /* device [n_prefill] state slots                 */
  const int32_t* decode_slots;  /* device [n_decode] state slots                  */
  const int32_t* block_tables;  /* device [n_prefill+n_decode][max_blocks_per_seq] */
  int max_blocks_per_seq;
  const int32_t* context_lens;  /* device [n_prefill+n_decode], new tokens included */
  const int32_t* cu_q_lens;     /* device [n_prefill+n_decode+1]: cu_seqlens, then +1 each */
  int max_context;              /* host bound on context_lens                     */
  int64_t n_blocks;             /* blocks in each full layer's pool               */
  int H;                        /* heads of linear layers = query heads of full layers */
  int H_kv;                     /* KV heads of full layers                        */
  int D;
  int chunk_size;               /* linear chunked prefill                         */
  float scale;                  /* softmax scale of full layers                   */
  hyattn_dtype dtype;
  void* workspace;              /* device, hyattn_hybrid_workspace_bytes() bytes  */
  size_t workspace_bytes;
} hyattn_batch;

size_t hyattn_hybrid_workspace_bytes(const hyattn_batch* batch);

/* layer_types: host int32[n_layers], each HYATTN_LAYER_LINEAR or _FULL; all
 * are checked before anything is launched (HYATTN_ERR_UNSUPPORTED_LAYER).
 * Linear layers are numbered 0, 1, ... in order of appearance and use that
 * layer of the state pool; each full layer uses its own k_pool/v_pool.
 * Per linear layer: chunked prefill of the prefill requests, then decode of
 * the decode requests. Per full layer: append the new K/V of every request,
 * causal prefill attention for the prefill requests, decode attention for
 * the decode requests. Launches go to `stream` in layer order, except that a
 * full layer with both prefill and decode requests runs its decode attention
 * on a second stream that the library keeps per device: forked from `stream`
 * after the append, joined back into `stream` (which waits for it) before the
 * next layer. Everything the step enqueues is thus complete once `stream`
 * reaches the point after the call. The fork and join are events, so the
 * step can be captured into a graph from `stream`; steps launched from
 * several host threads onto one device share that second stream and take
 * turns at each fork. */
hyattn_status hyattn_hybrid_step(const int32_t* layer_types, int n_layers,
                                 const hyattn_layer_io* layers, const hyattn_batch* batch,
                                 hyattn_state_pool* pool, void* stream);

/* ---------------------------------------------------------------------------
 * Memory estimate (page "推理框架适配Hybrid Model：KV Cache管理与算子调度实战",
 * §3.3 on sizing the two state kinds, §2.1 on what each layer type keeps):
 * device bytes a set of requests needs, for admission before any allocation.
 * Full layers keep K and V of every cached token (2 * L_full * H_kv * D *
 * elem_bytes per token); linear layers keep one H x D x D state per request
 * (L_lin * H * D * D * elem_bytes), whatever its length. Host only, no GPU.
 */
typedef struct {
  uint64_t kv_bytes;        /* 2 * L_full * H_kv * D * kv_elem_bytes * sum_r ctx_r      */
  uint64_t kv_paged_bytes;  /* the same with each context rounded up to 16-token blocks */
  uint64_t kv_blocks;       /* blocks one full layer's pool needs: sum_r ceil(ctx_r/16) */
  uint64_t state_bytes;     /* L_lin * H * D * D * n_requests * state_elem_bytes        */
  int n_full_layers;        /* layers of each type in layer_types                       */
  int n_linear_layers;
} hyattn_memory_estimate;

/* layer_types: host int32[n_layers] (HYATTN_LAYER_LINEAR / _FULL, anything
 * else is HYATTN_ERR_UNSUPPORTED_LAYER); context_lens: host int32[n_requests]
 * (tokens cached per request, >= 0); kv_elem_bytes / state_elem_bytes: bytes
 * per stored element (2 for bf16, 4 for fp32; this library stores states in
 * fp32, so its state pool is the state_elem_bytes = 4 figure). Negative or
 * inconsistent sizes, or a result beyond 2^64 - 1, give HYATTN_ERR_INVALID_ARG
 * and leave *out untouched. */
hyattn_status hyattn_estimate_memory(const int32_t* layer_types, int n_layers, int H, int H_kv,
                                     int D, const int32_t* context_lens, int n_requests,
                                     int kv_elem_bytes, int state_elem_bytes,
                                     hyattn_memory_estimate* out);

/* ---------------------------------------------------------------------------
 * Length-bucketed batch formation (page "推理框架适配Hybrid Model：KV Cache管理与
 * 算子调度实战", §2.4 on scheduling: a full layer's cost grows with the longest
 * sequence of its batch, a linear layer's does not, so requests of similar
 * length are batched together). Host only, no GPU.
 *
 * The cost of a batch is its padded size: requests x its longest length.
 * Requests are ordered by length (ties by index), and that order is cut into
 * consecutive batches, each taking requests while its padded size stays
 * <= max_padded_tokens and its request count <= max_requests. This gives the
 * fewest batches any grouping under the two limits can have (a grouping can
 * always be rearranged into consecutive runs of the sorted order without
 * raising any batch's longest length).
 *
 *   lengths           host int32[n]: tokens of each request (>= 0).
 *   max_padded_tokens per-batch limit on count * longest length (>= 1); a
 *                     single request longer than it is HYATTN_ERR_INVALID_ARG
 *                     (prefill such a request in chunks first).
 *   max_requests      per-batch limit on the request count (>= 1).
 *   order             host int32[n] out: request indices, batch by batch.
 *   batch_offsets     host int32[n+1] out: batch b holds
 *                     order[batch_offsets[b] .. batch_offsets[b+1]-1];
 *                     entries past *n_batches are left untouched.
 *   n_batches         host out: number of batches (0 for n = 0).
 * Invalid arguments give HYATTN_ERR_INVALID_ARG and leave the outputs
 * untouched. */
hyattn_status hyattn_bucket_by_length(const int32_t* lengths, int n, int64_t max_padded_tokens,
                                      int max_requests, int32_t* order, int32_t* batch_offsets,
                                      int* n_batches);

#ifdef __cplusplus
}
#endif
#endif /* HYATTN_H */
