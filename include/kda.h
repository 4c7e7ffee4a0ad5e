/*
 * kda.h - C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library.
 *
 * KDA is the per-head gated delta rule of "Kimi K3: KDA, Attention Residuals
 * and Stable LatentMoE" (hs-black.github.io/posts/kimi-k3):
 *   section 2.1  S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *                o_t = S_t^T q_t, q and k L2-normalised, computed in chunked form;
 *   section 2.2  alpha_t = e^{g_t},  g_t = g_min * Sigmoid(e^{A_h} z_t),  g_min = -5;
 *   section 2.3  y_t = Sigmoid(G_t) . RMSNorm(o_t)   (G_t = W_g x_t supplied by the caller;
 *                the W_g and W_o projections themselves are not part of this library).
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major, caller-owned DEVICE pointers (HIP device
 *    memory).  The library never allocates or frees device memory (apart from
 *    kda_chunk_fwd_noalloc's file-scope scratch array, see there).  Its only
 *    global state is per device: for the two-stream schedules of
 *    kda_chunk_fwd, one pair of library streams (default priority, each
 *    restricted to its own compute units; made by the first such call,
 *    rebuilt -- after waiting for them -- when a call needs a different
 *    split, released by kda_release_resources) and five events, guarded by a
 *    per-device lock.  It is safe to call from several host threads.
 *  - Hardware queues: the two-stream schedules use two queues of their own
 *    beside the caller's.  They do not depend on running concurrently for
 *    correctness (every producer launch is enqueued before the consumer that
 *    waits for it), only for speed.
 *  - Layouts: q, k, z: [B, T, H, d_k]; v, o, gate, y: [B, T, H, d_v];
 *    beta: [B, T, H] (or head first, [B, H, T, ..], see kda_token_layout);
 *    A: [H] fp32; states S0, S_T, S_pool: [.., H, d_k, d_v] fp32 with the key
 *    channel as row index (o = S^T q).
 *  - Element types: q, k, v, beta, z and gate are all `in_dtype`; o and y are
 *    `out_dtype`; A, states and rms_w are fp32.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and returns without waiting for the GPU.
 *  - Errors: arguments are validated on the host before anything is enqueued.
 *    On any error nothing is enqueued and no output is touched.  A failed
 *    kernel launch returns KDA_ERR_HIP.  No C++ exception crosses the ABI.
 *  - Pointers to q, k, v, z, gate, o, y and to the workspace must be 16-byte
 *    aligned; beta 2-byte (bf16) or 4-byte (fp32); A, rms_w, S0, S_T, S_pool
 *    4-byte.
 *  - Supported shapes: d_k == d_v in {64, 128}, chunk == 64, B, H >= 1, T >= 0,
 *    any T (a short last chunk is handled), -5.5 <= g_min < 0 (so a 16-token
 *    sub-tile's cumulative log-decay stays above -88, keeping its reciprocal
 *    within bf16 / fp32 range, section 2.2).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 6

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL_ARG = 1,     /* a required pointer is NULL                         */
  KDA_ERR_BAD_SHAPE = 2,    /* a size is negative / zero where it must not be      */
  KDA_ERR_BAD_DTYPE = 3,    /* unknown dtype enum                                  */
  KDA_ERR_MISALIGNED = 4,   /* a pointer breaks the alignment rules above          */
  KDA_ERR_UNSUPPORTED = 5,  /* valid request outside what the kernels implement    */
  KDA_ERR_WORKSPACE = 6,    /* workspace missing or smaller than one chunk needs   */
  KDA_ERR_HIP = 7,          /* a kernel launch failed (HIP error read and cleared)  */
  KDA_ERR_TIMEOUT = 8       /* reported by kda_chunk_fwd_status: an in-kernel wait
                               for chunk records gave up (outputs are invalid)     */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum { KDA_STATE_ZERO = 0, KDA_STATE_IMPORT = 1, KDA_STATE_EXPORT = 2 } kda_state_op;

/* Decay maps.  KDA_DECAY_K3 is the method (section 2.2): g = g_min
 * Sigmoid(e^{A_h} z), bounded below.  KDA_DECAY_SOFTPLUS is Kimi Linear's
 * g = -e^{A_h} Softplus(z), the unbounded map section 2.2 replaces, kept as
 * an ablation: without the bound the diagonal 16-token blocks are computed
 * pair by pair (slower), which is what the bound removes. */
typedef enum { KDA_DECAY_K3 = 0, KDA_DECAY_SOFTPLUS = 1 } kda_decay;

/* Schedules of kda_chunk_fwd (see there). */
typedef enum {
  KDA_SCHEDULE_SEGMENTS = 0,   /* intra-chunk kernel, then scan, segment after segment */
  KDA_SCHEDULE_OVERLAPPED = 1, /* the two kernels of consecutive segments overlapped   */
  KDA_SCHEDULE_FUSED = 2,      /* one fused kernel, chunk records kept in LDS          */
  KDA_SCHEDULE_PIPELINED = 3   /* every record in the workspace: one intra-chunk launch
                                  beside one scan launch over the sequence            */
} kda_schedule;

/* Kernel launches that kda_chunk_fwd_traced times (kda_chunk_fwd_launches). */
typedef enum { KDA_LAUNCH_INTRA = 0, KDA_LAUNCH_SCAN = 1, KDA_LAUNCH_FUSED = 2 } kda_launch_kind;

/* Order of the per-token tensors of kda_chunk_fwd* (q, k, z, v, gate, o, y:
 * [B, T, H, d] or [B, H, T, d]; beta: [B, T, H] or [B, H, T]); the innermost
 * d elements are contiguous either way.  kda_prepass and kda_input_prep take
 * token major only (KDA_ERR_UNSUPPORTED for KDA_TOKENS_BHTD).  Token
 * major is what a projection of the hidden state writes directly; head
 * first puts each head's tokens in one block, so that the 64 rows of a
 * chunk are one contiguous 16 KB (bf16, d = 128) instead of 64 rows a token
 * stride apart, which the state scan reads and writes faster beside the
 * intra-chunk kernel. */
typedef enum { KDA_TOKENS_BTHD = 0, KDA_TOKENS_BHTD = 1 } kda_token_layout;

typedef enum {
  KDA_LAYOUT_KV = 0, /* user state is [d_k][d_v], same as the pool               */
  KDA_LAYOUT_VK = 1  /* user state is [d_v][d_k] (transposed)                      */
} kda_state_layout;

/* Problem descriptor.  kda_desc_init fills the defaults shown. */
typedef struct {
  int32_t B, T, H;       /* batch, tokens per sequence, heads                      */
  int32_t d_k, d_v;      /* head dims (equal; 64 or 128)                           */
  int32_t chunk;         /* tokens per chunk: 64                                   */
  float g_min;           /* lower bound of the log-decay: -5                       */
  float q_scale;         /* multiplier of q after L2Norm: 1 (the pages show none)  */
  float l2_eps;          /* q / sqrt(|q|^2 + l2_eps): 1e-6                          */
  float rms_eps;         /* o / sqrt(mean(o^2) + rms_eps): 1e-6                     */
  int32_t qk_l2norm;     /* 1: L2-normalise q and k inside the kernel               */
  kda_dtype in_dtype;    /* q, k, v, beta, z, gate                                 */
  kda_dtype out_dtype;   /* o, y                                                   */
  int32_t segment_tokens; /* tokens per internal segment of the overlapped
                             and pipelined schedules; 0: library default
                             (8192 overlapped, 128 pipelined)                */
  int32_t overlap;       /* 1: run the intra-chunk kernel of the next segment
                            concurrently with the scan of the current one
                            (library-owned streams, see kda_chunk_fwd); 0: one
                            stream, segments in turn                          */
  int32_t fused;         /* the fused one-kernel schedule (bf16 inputs, K3
                            decay only): 2 forces it; 1 (default) lets the
                            library choose, which currently always takes the
                            two-kernel schedules (measured faster); 0 never */
  kda_decay decay;       /* decay map: KDA_DECAY_K3 (default) or the
                            KDA_DECAY_SOFTPLUS ablation; used by
                            kda_chunk_fwd*, kda_recurrent_step, kda_prepass;
                            g_min applies to the K3 map only                  */
  kda_token_layout tokens; /* order of the per-token tensors (above):
                            KDA_TOKENS_BTHD (default) or KDA_TOKENS_BHTD;
                            kda_recurrent_step (one token) ignores it        */
} kda_desc;

/* ABI version of the loaded library (KDA_ABI_VERSION it was built with). */
int kda_abi_version(void);

/* Static description of a status code. */
const char* kda_status_str(kda_status s);

/* Fill *d with the defaults above for the given sizes and dtypes. */
kda_status kda_desc_init(kda_desc* d, int32_t B, int32_t T, int32_t H, int32_t head_dim, kda_dtype in_dtype,
                         kda_dtype out_dtype);

/* Workspace bytes for kda_chunk_fwd's preferred schedule; 0 if *d is invalid.
 * The fused schedule needs none (256 is reported; ws may also be NULL then).
 * With d->overlap, bf16 inputs and a sequence longer than 8,192 tokens this
 * holds every chunk record of the call (the pipelined schedule: 61,952 bytes
 * per chunk and (b, h) at d = 128, e.g. 6.1 GB for B 1, T 65,536, H 96) as
 * long as that is at most 8 GiB, and otherwise the largest window of the
 * pipelined schedule within 8 GiB (e.g. 1,444 chunks = 92,416 tokens for
 * H 96); else the whole sequence (at most 65536 tokens per segment).  A
 * smaller workspace also works as long as it holds one chunk: the library
 * takes the pipelined schedule in windows if at least 512 chunks of records
 * fit, else the overlapped schedule if two segments of d->segment_tokens
 * (default 8192) fit, else it processes the sequence in shorter segments,
 * one after the other. */
size_t kda_chunk_fwd_workspace_size(const kda_desc* d);

/* Bytes needed for one segment of `segment_tokens` tokens (rounded up to whole
 * chunks) processed in turn; 0 if *d is invalid. */
size_t kda_chunk_fwd_workspace_size_for(const kda_desc* d, int32_t segment_tokens);

/*
 * Waits for and destroys the streams and events the two-stream schedules
 * created (on every device); later calls create them again.  Optional: call
 * before the process or the HIP runtime shuts down when tools that track
 * queues (profilers) are attached.  Not thread-safe against concurrent calls
 * of kda_chunk_fwd.
 */
kda_status kda_release_resources(void);

/*
 * The schedule kda_chunk_fwd takes on the current device for this descriptor
 * and a workspace of ws_bytes bytes: *segment_tokens receives the tokens per
 * segment (a multiple of the chunk; the whole sequence for the fused
 * schedule, the record-counting segment for the pipelined one), *schedule a
 * kda_schedule value.  KDA_ERR_WORKSPACE if a
 * two-kernel schedule is taken and the workspace is too small for one chunk.
 */
kda_status kda_chunk_fwd_schedule(const kda_desc* d, size_t ws_bytes, int32_t* segment_tokens,
                                  int32_t* schedule);

/*
 * Outcome of the most recent kda_chunk_fwd / kda_chunk_fwd_traced call that
 * used workspace ws (ws_bytes bytes) with this descriptor: waits for `stream`
 * (a host synchronisation, unlike every other entry point), then returns
 * KDA_OK, or KDA_ERR_TIMEOUT when that call took a two-stream schedule and
 * one of the scan's bounded in-kernel waits gave up -- for chunk records
 * whose producers never ran beside it, or, in the one-stream schedule with
 * a head's scan split between two workgroups, for the other workgroup (e.g.
 * another process held the device's compute units for about a second); the
 * call's outputs are then invalid (NaN).  Calls that took the fused
 * schedule, or the one-stream schedule without the split, always report
 * KDA_OK here.
 */
kda_status kda_chunk_fwd_status(const kda_desc* d, const void* ws, size_t ws_bytes, void* stream);

/* The kernel launches, in order, that kda_chunk_fwd_traced brackets with
 * events for this descriptor and workspace size on the current device:
 * *n_launches receives their number and kinds[i] (i < max_kinds) the
 * kda_launch_kind of the i-th.  Segments and overlapped: per segment the
 * intra-chunk kernel, then the scan; pipelined: the intra-chunk kernel (one
 * launch), then the scan (one launch); fused: one launch.  kinds may be NULL when max_kinds is 0. */
kda_status kda_chunk_fwd_launches(const kda_desc* d, size_t ws_bytes, int32_t* kinds, int32_t max_kinds,
                                  int32_t* n_launches);

/*
 * Chunked KDA forward over whole sequences (prefill / training forward),
 * section 2.1's chunk form with section 2.2's 16-token dense sub-tiles.
 *
 *  q, k, v, beta, z, A   inputs (see layouts above); beta in (0, 1).
 *         The shapes here are token major; with d->tokens ==
 *         KDA_TOKENS_BHTD every [B, T, H, ..] below is [B, H, T, ..].
 *  S0     [B, H, d_k, d_v] fp32 initial state, or NULL for zero.
 *  gate   [B, T, H, d_v] gate logits W_g x, or NULL (no gate).
 *  rms_w  [H, d_v] fp32 RMSNorm weight, or NULL (weight 1).
 *  o      [B, T, H, d_v] output o_t = S_t^T q_t, or NULL.
 *  y      [B, T, H, d_v] gated output (requires gate), or NULL.
 *  S_T    [B, H, d_k, d_v] fp32 final state, or NULL.  May alias S0.
 *  ws     device workspace of ws_bytes bytes (see the size queries), owned by
 *         the caller; its contents are scratch.  May be NULL when T == 0 or
 *         when the fused schedule is taken.
 * At least one of o, y, S_T must be non-NULL.  o, y and S_T must not overlap
 * any input or each other, except S_T == S0 (KDA_ERR_UNSUPPORTED otherwise).
 * When d->T == 0 nothing is read:
 * S_T receives S0 (or zeros) and q, k, v, beta, z, A and ws may be NULL.
 *
 * Fused schedule (d->fused == 2; bf16 inputs, K3 decay): one launch, one
 * workgroup per (head, sequence).  Its compute waves run the state scan of
 * chunk c while producer waves build chunk c + 1's intra-chunk record
 * directly in LDS and write chunk c - 1's o / y, so no record goes through
 * HBM.  Each head's intra-chunk work then runs on a single compute unit,
 * which measured slower than the two-kernel schedules at every size tried.
 * Results are bit-identical to the two-kernel schedules.
 *
 * Two-kernel schedules.  The sequence is processed in segments; per segment the
 * intra-chunk kernel writes one record per chunk into the workspace and the
 * state scan (with the fused gate) consumes them.  When d->overlap is set, the
 * sequence spans more than one segment of d->segment_tokens tokens, B * H is
 * at most 5/8 of the device's compute units and the workspace holds two
 * segments, the work runs on two library-owned streams of the current device
 * (created on first use, default priority, each restricted to its own set of
 * compute units): the intra-chunk kernel of segment s + 1 runs while the scan
 * of segment s runs, with HIP events ordering both against `stream` at the
 * start and the end of the call.  The call still behaves as one operation
 * enqueued on `stream`.  Calls that overlap in time on one device serialise
 * their enqueue (a per-device lock); they must not share a workspace.
 *
 * Pipelined schedule (the same conditions, bf16 inputs, and a workspace that
 * holds every chunk record of the call, or at least 512 chunks of them: the
 * sequence is then processed in windows of as many whole segments as fit,
 * the state carried from window to window and each window's producers
 * waiting for the previous window's scan through an event): per window one
 * intra-chunk launch runs on one library stream, producing the records chunk
 * by chunk (every head's record of chunk c before any of chunk c + 1), and a
 * single scan launch over the window runs on the other, waiting
 * inside the kernel for each segment's records (device-scope record stores,
 * one counter per segment and (b, h); segments of d->segment_tokens tokens,
 * 128 by default).  The scan publishes each (b, h)'s chunk every step, and
 * every second chunk's producers wait until their scan is within a segment
 * plus six chunks, so that records are read back from the memory-side cache; this pacing is a bounded wait that switches itself off
 * for the call when it runs out, and never affects results.  The
 * intra-chunk launch is enqueued before the scan, so
 * the call completes correctly even when the two library streams
 * end up sharing a hardware queue (their work then runs one after the
 * other).  The waits are bounded (about a second): a producer kept from
 * running that long shows as NaN output, not a hang, and
 * kda_chunk_fwd_status reports KDA_ERR_TIMEOUT for the call.  Results are
 * bit-identical to the other two-kernel schedules.
 *
 * When `stream` is being captured into a HIP graph, the one-stream schedule
 * is taken (its launches have no in-kernel waits on other nodes).
 */
kda_status kda_chunk_fwd(const kda_desc* d, const void* q, const void* k, const void* v, const void* beta,
                         const void* z, const float* A, const float* S0, const void* gate, const float* rms_w,
                         void* o, void* y, float* S_T, void* ws, size_t ws_bytes, void* stream);

/* Size of the device scratch array kda_chunk_fwd_noalloc works in (per GPU). */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * kda_chunk_fwd without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, results and errors as kda_chunk_fwd, minus
 * ws / ws_bytes.  It always takes the one-stream schedule (segments in turn
 * on `stream`, so no library streams or events either) and keeps its chunk
 * records and the carried state in a file-scope device array of
 * KDA_NOALLOC_SCRATCH_BYTES bytes, which every GPU the library runs on holds
 * until the process ends (its address is resolved on the first call on each
 * device).  It calls no hipMalloc, hipFree or other allocating routine.
 *  - The sequence is processed in segments of as many chunks as the array
 *    holds; a call whose single chunk does not fit (B * H * (one chunk record
 *    + one fp32 state) above the limit: B * H > ~1000 at d = 128) returns
 *    KDA_ERR_WORKSPACE and enqueues nothing.
 *  - Every call on one GPU shares that GPU's array: calls that can overlap in
 *    time on one device (several streams, several host threads) race and
 *    must be serialised by the caller.  Nothing in the array needs to start
 *    zeroed; each call overwrites what it reads.
 */
kda_status kda_chunk_fwd_noalloc(const kda_desc* d, const void* q, const void* k, const void* v, const void* beta,
                                 const void* z, const float* A, const float* S0, const void* gate,
                                 const float* rms_w, void* o, void* y, float* S_T, void* stream);

/*
 * kda_chunk_fwd with per-kernel timing: identical work and results, and in
 * addition, for the i-th kernel launch of the call (the order that
 * kda_chunk_fwd_launches reports),
 * hipEventRecord(events[2i]) right before it and hipEventRecord(events[2i+1])
 * right after it on the stream that launch uses (`stream`, or the library's
 * stream of that kernel in the overlapped schedule), while 2i+1 < n_events.
 * `events` are caller-owned hipEvent_t handles.  Used to measure kernel
 * durations on the launch stream.
 */
kda_status kda_chunk_fwd_traced(const kda_desc* d, const void* q, const void* k, const void* v, const void* beta,
                                const void* z, const float* A, const float* S0, const void* gate,
                                const float* rms_w, void* o, void* y, float* S_T, void* ws, size_t ws_bytes,
                                void* stream, void* const* events, int32_t n_events);

/*
 * Prefix-cache snapshots: kda_chunk_fwd plus the recurrent state at every
 * `every_chunks`-th chunk boundary (K3 blog section 13.1: a cached prefix of
 * a KDA layer is reusable only as the state at a chunk-aligned boundary).
 * snapshots is fp32 [B, n, H, d_k, d_v] with n = kda_snapshot_count(d,
 * every_chunks) = floor(T / (64 * every_chunks)); snapshot j of sequence b is
 * the state after token (j + 1) * 64 * every_chunks - 1, i.e. the S0 with
 * which a forward over the remaining tokens resumes (bit-identically).
 * o, y and S_T may all be NULL here (then n == 0 does nothing and
 * snapshots may be NULL whenever n == 0).  The snapshots share the forward's
 * launches: each scan workgroup stores its head's state (64 KiB at d = 128)
 * when it crosses a snapshot boundary.  KDA_ERR_BAD_SHAPE if
 * every_chunks < 1.
 */
kda_status kda_chunk_fwd_snapshots(const kda_desc* d, const void* q, const void* k, const void* v,
                                   const void* beta, const void* z, const float* A, const float* S0,
                                   const void* gate, const float* rms_w, void* o, void* y, float* S_T,
                                   float* snapshots, int32_t every_chunks, void* ws, size_t ws_bytes, void* stream);

/* Number of snapshots kda_chunk_fwd_snapshots writes per sequence (0 if *d is
 * invalid or every_chunks < 1). */
int32_t kda_snapshot_count(const kda_desc* d, int32_t every_chunks);

/*
 * kda_chunk_fwd with the sequence cut into n_parts equal segments that are
 * processed in parallel (KCP, K3 blog section 10.2, on one GPU): over a
 * segment the state map is affine, S_out = M S_in + S~.  Pass 1 runs every
 * segment at once from S = I with V = 0 (giving M) and from S = 0 (giving
 * S~); a fold along each sequence gives every segment's entry state
 * (S_in[p + 1] = M[p] S_in[p] + S~[p], S_in[0] = S0); pass 2 runs every
 * segment at once from its entry state and writes o / y.  S_T is pass 2's
 * state after the last segment.  Arguments as kda_chunk_fwd; ws of
 * kda_chunk_fwd_kcp_workspace_size(d, n_parts) bytes (three fp32 state sets
 * of B * n_parts * H * d_k * d_v plus the segments' own workspace).
 * T must be a multiple of 64 * n_parts and the tensors token major
 * (KDA_ERR_UNSUPPORTED otherwise);
 * n_parts == 1 is kda_chunk_fwd.  Outputs equal kda_chunk_fwd's up to fp32
 * rounding of the folded entry states.  The work is about three forward
 * passes: this is the one-GPU share of sequence parallelism across GPUs, not
 * a faster single-GPU schedule.
 */
kda_status kda_chunk_fwd_kcp(const kda_desc* d, int32_t n_parts, const void* q, const void* k, const void* v,
                             const void* beta, const void* z, const float* A, const float* S0, const void* gate,
                             const float* rms_w, void* o, void* y, float* S_T, void* ws, size_t ws_bytes,
                             void* stream);

/* Workspace bytes for kda_chunk_fwd_kcp (0 if *d is invalid or T is not a
 * multiple of 64 * n_parts, or the tensors are head first). */
size_t kda_chunk_fwd_kcp_workspace_size(const kda_desc* d, int32_t n_parts);

/*
 * Input steps before the core (K3 blog section 2.1): from the projections
 * x_q, x_k, x_v [B, T, H, d] and the beta logits [B, T, H] (all d->in_dtype),
 *     q = Swish(ShortConv(x_q)),  k = Swish(ShortConv(x_k)),
 *     v = Swish(ShortConv(x_v)),  beta = Sigmoid(beta_logits),
 * written to q, k, v [B, T, H, d] and beta [B, T, H] in d->in_dtype; Swish(x)
 * = x Sigmoid(x).  The L2Norm of q and k is applied by kda_chunk_fwd /
 * kda_recurrent_step (d->qk_l2norm), not here.  ShortConv is a depthwise
 * causal convolution over time with conv_width (1..4) taps per channel and no
 * bias (the pages give neither a width nor a bias): wq, wk, wv are fp32
 * [H * d, conv_width], tap conv_width - 1 multiplying the current token and
 * tap conv_width - 1 - j the token j steps back.
 *  state_in   fp32 [B, 3, conv_width - 1, H * d]: the conv_width - 1 inputs
 *             of q, k, v (in that order) before token 0, oldest first; NULL
 *             for zeros (the start of a sequence).
 *  state_out  same layout: receives the conv_width - 1 inputs before token T
 *             (the state a later call, e.g. a decode step with T = 1,
 *             continues from); NULL to skip.  May equal state_in (the
 *             sequence is then processed in one block of tokens per channel
 *             group: fine for decode, slow for long prefills).
 *  beta_logits, beta  both NULL to skip beta.
 * With T == 0 only state_out is written (state_in copied, or zeros).
 * Outputs must not overlap the inputs or each other, except beta ==
 * beta_logits and state_out == state_in (KDA_ERR_UNSUPPORTED otherwise: a
 * block of tokens re-reads the inputs just before it).
 * KDA_ERR_UNSUPPORTED if conv_width is outside 1..4.  Chaining calls through
 * the state gives the same outputs as one call over the concatenated tokens.
 */
kda_status kda_input_prep(const kda_desc* d, int32_t conv_width, const void* xq, const void* xk, const void* xv,
                          const void* beta_logits, const float* wq, const float* wk, const float* wv,
                          const float* state_in, float* state_out, void* q, void* k, void* v, void* beta,
                          void* stream);

/* Bit that kda_recurrent_step / kda_state_io OR into *status for a slot
 * outside [0, n_slots) (that sequence / state is skipped, nothing of it is
 * read or written). */
#define KDA_FLAG_BAD_SLOT 1u

/*
 * One decode step (single token) for d->B sequences: the same recurrence,
 * section 2.1, applied to one token.  d->T must be 1.  Each sequence n reads
 * and updates its state in place at S_pool[slot[n]] (slot == NULL: slot n):
 *  q, k, v, z, gate, o, y  are [B, 1, H, d], beta is [B, 1, H];
 *  S_pool  [n_slots, H, d_k, d_v] fp32 state pool, updated in place;
 *  slot    [B] int32 device array of distinct pool rows, or NULL (then
 *          B <= n_slots, else KDA_ERR_BAD_SHAPE);
 *  o, y    outputs as in kda_chunk_fwd (y requires gate);
 *  status  device uint32 or NULL: a sequence whose slot lies outside
 *          [0, n_slots) is skipped (its state row, o and y are not touched)
 *          and KDA_FLAG_BAD_SLOT is OR-ed into *status (which the caller
 *          clears).  The slots live in device memory, so this check runs in
 *          the kernel, not on the host.
 * Slots must be distinct within one call (two sequences writing one slot race).
 */
kda_status kda_recurrent_step(const kda_desc* d, const void* q, const void* k, const void* v, const void* beta,
                              const void* z, const float* A, float* S_pool, int32_t n_slots, const int32_t* slot,
                              const void* gate, const float* rms_w, void* o, void* y, uint32_t* status,
                              void* stream);

/*
 * State hand-off between a state pool and caller buffers (prefill -> decode,
 * prefix-cache snapshots): ZERO clears pool rows, IMPORT copies user -> pool,
 * EXPORT copies pool -> user.
 *  n      number of states moved; slot [n] int32 device array or NULL (0..n-1,
 *         then n <= n_slots);
 *  pool   [n_slots, H, d_k, d_v] fp32;  user [n, H, ...] fp32 in `layout`
 *         (NULL for ZERO).  d_k == d_v in {64, 128}.
 *  status device uint32 or NULL: a slot outside [0, n_slots) is skipped and
 *         KDA_FLAG_BAD_SLOT is OR-ed into *status, as for kda_recurrent_step.
 */
kda_status kda_state_io(kda_state_op op, int32_t n, int32_t H, int32_t d_k, int32_t d_v, kda_state_layout layout,
                        float* pool, int32_t n_slots, const int32_t* slot, float* user, uint32_t* status,
                        void* stream);

/*
 * Pre-pass diagnostic (the first step of kda_chunk_fwd, exposed for tests):
 *  G      [B, T, H, d_k] fp32, chunk-local inclusive cumulative sum of
 *         g = g_min * Sigmoid(e^{A_h} z) over each 64-token chunk (section 2.2);
 *  rq, rk [B, T, H] fp32 inverse L2 norms 1 / sqrt(|x|^2 + l2_eps) (1 when
 *         d->qk_l2norm == 0).
 */
kda_status kda_prepass(const kda_desc* d, const void* q, const void* k, const void* z, const float* A, float* G,
                       float* rq, float* rk, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
