/*
 * blk.h -- C ABI of the MI355X (gfx950) block-stage library `libblk.so`.
 *
 * One transformer-block stage runs on a small chunk of query tokens that
 * reads a cached prefix / history K/V.  The same stage, repeated over a layer
 * stack and a flow-matching Euler loop, is an action expert's denoise step.
 *
 * Sources for what is computed:
 *   [PS] AREX Feed article on PhysisServe: a pipeline stage is one Transformer
 *        block at one denoise step; a chunk reads the cached (noisy) KV of
 *        earlier chunks; the KV cache stays on its GPU; only hidden states
 *        move between stages (section on splitting the pipeline per block
 *        and step).
 *   [RT] reading note on "Running VLAs at Real-time Speed" (Ma et al.,
 *        arXiv:2510.26742v1): RMSNorm gain folded into the next linear layer
 *        (§4.1); action and time-embedding linears pre-multiplied, the time
 *        branch tabulated for fixed timesteps and folded into the bias ahead
 *        of SiLU (§4.2); Q/K/V merged into one matrix with RoPE fused into
 *        the product (§4.3); gated FFN, bias/residual/activation epilogues
 *        and precomputed RMS statistics (§5); graph capture of a fixed
 *        sequence of GPU work with stable shapes and addresses (§3).
 *   [TR] TileRT article: at decode-sized work the gaps between kernels
 *        (launches, barriers, memory round trips) dominate; one resident
 *        kernel runs the operator sequence as tile tasks.
 *
 * Conventions for every call:
 *   - Matrices are row-major [in, out] (row-vector convention y = x W).
 *   - bf16 tensors are passed as their 16-bit patterns (uint16_t).  Gains,
 *     biases, tables, noise, state and actions are float32.
 *   - Every pointer named "device" is device memory owned by the caller; the
 *     library never frees or retains caller memory beyond the call, except
 *     that flow_denoise's captured graph keeps the pointers of its key
 *     (see flow_denoise).  The library allocates no device memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and is asynchronous; no call synchronizes the device except
 *     flow_denoise while it captures a new graph.
 *   - Return value 0 = success, negative = one of the BLK_E* codes below.
 *     All arguments are validated before anything is enqueued; on error
 *     nothing is enqueued and blk_last_error() returns a message (per
 *     calling thread).  No call aborts or throws.
 *   - Size-query protocol: a call whose output buffer pointer is NULL only
 *     writes the required byte count to *bytes / *ws_bytes and returns 0.
 *   - Calls sharing a workspace must not overlap in time (same stream is
 *     fine).  A workspace must be zero-filled before its first use.  Its
 *     first BLK_WS_SYNC_BYTES bytes are a synchronization region laid out the
 *     same way for every config and entry point (arrival counters, which
 *     every call leaves at zero, and monotonic phase flags); activations and
 *     partials follow it.  So one workspace, large enough for each call, may
 *     serve blk_forward and flow_denoise calls of different shapes in turn.
 */
#ifndef BLK_H_
#define BLK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BLK_OK 0
#define BLK_EINVAL (-1)       /* NULL pointer, negative size, out-of-range index      */
#define BLK_EUNSUPPORTED (-2) /* shape outside the supported set                     */
#define BLK_ESIZE (-3)        /* a buffer is smaller than its size query              */
#define BLK_ESTATE (-4)       /* packed buffer unknown, or config/steps do not match */
#define BLK_EHIP (-5)         /* a HIP runtime call failed (message has the reason)  */
#define BLK_EABORTED (-6)     /* a persistent launch on this workspace timed out     */

/* Size of the synchronization region at the start of every workspace, and the
 * byte offset of its abort word (see blk_set_execution_mode). */
#define BLK_WS_SYNC_BYTES 110848
#define BLK_WS_ABORT_OFFSET 110600

/* Shape of one block.  Supported: head_dim in {64, 128, 256}; hidden % 128 == 0;
 * ffn % 128 == 0; n_q_heads % n_kv_heads == 0; 1 <= max_pos <= 1<<20. */
typedef struct blk_config {
  int32_t hidden;      /* D: model width                                         */
  int32_t ffn;         /* F: gated-FFN width                                      */
  int32_t n_q_heads;   /* Hq                                                      */
  int32_t n_kv_heads;  /* Hkv (Hq == Hkv: MHA; Hkv == 1: MQA); head h reads kv-head
                          floor(h * Hkv / Hq)                                     */
  int32_t head_dim;    /* d                                                       */
  int32_t max_pos;     /* RoPE table length: every position P + t must be < max_pos */
  float rope_base;     /* theta_j = rope_base^(-2j/d), pairs (j, j + d/2)         */
  float rms_eps;       /* RMSNorm: x * (mean x^2 + eps)^-1/2 * g                  */
} blk_config;

/* One layer's raw (unfolded) weights, all device pointers. */
typedef struct blk_layer_src {
  const float* g_attn;     /* [D]          RMSNorm gain ahead of attention          */
  const uint16_t* w_q;     /* bf16 [D][Hq*d]                                        */
  const uint16_t* w_k;     /* bf16 [D][Hkv*d]                                       */
  const uint16_t* w_v;     /* bf16 [D][Hkv*d]                                       */
  const uint16_t* w_o;     /* bf16 [Hq*d][D]                                        */
  const float* g_ffn;      /* [D]          RMSNorm gain ahead of the FFN            */
  const uint16_t* w_gate;  /* bf16 [D][F]                                           */
  const uint16_t* w_up;    /* bf16 [D][F]                                           */
  const uint16_t* w_down;  /* bf16 [F][D]                                           */
} blk_layer_src;

/* Flow-matching head of an action expert ([RT] §2, §4.2), device pointers. */
typedef struct blk_flow_head_src {
  int32_t n_actions;       /* N action tokens (the chunk is N + 1 tokens: state first) */
  int32_t action_dim;      /* A (<= 64)                                              */
  const uint16_t* w1;      /* bf16 [A][D]   action projection                        */
  const float* b1;         /* [D]                                                    */
  const uint16_t* w2;      /* bf16 [2D][D]  rows 0..D-1: action branch, D..2D-1: time */
  const float* b2;         /* [D]                                                    */
  const uint16_t* w3;      /* bf16 [D][D]   linear after SiLU                        */
  const float* b3;         /* [D]                                                    */
  const uint16_t* ws;      /* bf16 [A][D]   state projection                         */
  const float* bs;         /* [D]                                                    */
  const float* g_f;        /* [D]           final RMSNorm gain                       */
  const uint16_t* w_out;   /* bf16 [D][A]   velocity projection                      */
  const float* b_out;      /* [A]                                                    */
} blk_flow_head_src;

/*
 * blk_prepare_weights -- the weight-prep pass ([RT] §4.1-4.3), once per model.
 *
 * Packs n_layers layers (host array `layers` of device pointers) and, if
 * `head` is non-NULL, a flow head for the n_steps evaluation times
 * t_schedule[0..n_steps-1] (host float64 array) into one opaque device buffer
 * `dst`:
 *   - RMSNorm gains folded into the following projection: diag(g) W, product
 *     formed exactly and rounded once to bf16;
 *   - W_q | W_k | W_v concatenated into one matrix, columns regrouped so the
 *     RoPE pair (j, j + d/2) of every rotated head is produced together;
 *     W_gate and W_up interleaved per 16-column tile; all matrices stored as
 *     MFMA operand fragments;
 *   - RoPE cos/sin table [max_pos][d/2] (float64 math, float32 storage);
 *   - flow head: W1 W2a (float32), bias table b1 W2a + tau(t_s) W2t + b2 per
 *     step (float32; tau is the sinusoidal embedding of t_s), Euler steps
 *     t_{s+1} - t_s (t_{n_steps} = 0), final gain folded into W_out.
 * The table depends on the schedule: a different schedule needs a new prepare.
 * dst == NULL: only *bytes is set.  Otherwise *bytes must be >= the query.
 * The source buffers must stay valid until the enqueued work has run; dst is
 * registered in a host-side table (keyed by address) that blk_forward and
 * flow_denoise consult.  Errors: BLK_EINVAL, BLK_EUNSUPPORTED, BLK_ESIZE,
 * BLK_EHIP.
 */
int blk_prepare_weights(const blk_config* cfg, const blk_layer_src* layers, int n_layers,
                        const blk_flow_head_src* head, const double* t_schedule, int n_steps,
                        void* dst, size_t* bytes, void* stream);

/*
 * blk_forward -- one block stage over cached K/V ([PS]; [RT] §4-§5).
 *
 * For each of `batch` streams b (all on the same layer weights, [PS] batching
 * of one block's tasks across chunks), with T = tokens, P = prefix:
 *   x       device bf16 [batch][T][D]           chunk hidden states (input)
 *   k_prefix, v_prefix  device bf16, stream b at element offset
 *           b * prefix_stride, each [P][Hkv][d]  cached keys (already rotated)
 *           and values; read only; may be NULL when P == 0; prefix_stride 0
 *           makes every stream read the same prefix
 *   y       device bf16 [batch][T][D]           block output
 *   k_new, v_new  device bf16, stream b at b * new_stride, each [T][Hkv][d]:
 *           the chunk's own keys (after RoPE) and values.  They may alias
 *           rows P..P+T-1 of the caller's cache (k_new = k_prefix + P*Hkv*d,
 *           new_stride = prefix_stride) to append the chunk to the cache.
 *   ws      device workspace of *ws_bytes bytes (query with ws == NULL);
 *           zero-filled before its first use.
 * x, y, k_new, v_new, k_prefix and v_prefix must be 16-byte aligned and both
 * strides multiples of 8 elements (the kernels move 16-byte vectors).
 * Computes y = h + FFN(RMSNorm(h) g2), h = x + Attn(RoPE(Q), [K_p; RoPE(K)],
 * [V_p; V]) W_o with Q, K, V = RMSNorm(x) g1 [W_q|W_k|W_v]; chunk token t is at
 * position P + t; no attention mask (every query sees all P + T keys).
 * `packed` must come from blk_prepare_weights with an identical cfg; `layer`
 * selects the layer.  Errors: BLK_EINVAL (also misaligned buffers or strides),
 * BLK_EUNSUPPORTED (P + T > max_pos; batch * tokens * max(hidden, ffn, Hq d)
 * above 2^30),
 * BLK_ESIZE (ws too small), BLK_ESTATE (packed unknown / cfg differs), BLK_EHIP.
 */
int blk_forward(const blk_config* cfg, const void* packed, int layer, int batch, int tokens,
                int prefix, const uint16_t* x, const uint16_t* k_prefix,
                const uint16_t* v_prefix, int64_t prefix_stride, uint16_t* y, uint16_t* k_new,
                uint16_t* v_new, int64_t new_stride, void* ws, size_t* ws_bytes, void* stream);

/*
 * blk_forward_chunks -- blk_forward for a batch of chunks whose histories
 * differ in length: the same-block batch of chunks at different points of a
 * chunk-autoregressive schedule, each reading the cached (noisy) K/V written
 * before it and producing its own ([PS], sections on the pipeline per denoise
 * step and block and on same-block batching across chunks).
 *
 * Same arguments, layouts, results and errors as blk_forward, plus
 *   prefix_lens  host int32 [batch]: stream b attends to the first
 *                prefix_lens[b] rows of its prefix (0 <= prefix_lens[b] <= P,
 *                P = prefix sizes the buffers and the workspace) and to its
 *                own T keys, and its token t is at position prefix_lens[b] + t.
 * With prefix_stride 0 every stream reads the first rows of one shared cache
 * (a stream's K_new / V_new may then be appended to it for the next call; a
 * call never reads what it writes).  Streams with prefix_lens[b] == P give
 * exactly blk_forward's result.  The array is read during the call only.
 * Runs on the per-operator kernels (BLK_EUNSUPPORTED when execution mode 2
 * forces the persistent kernel).  Errors as blk_forward, plus BLK_EINVAL
 * (prefix_lens NULL with batch > 0, or a length outside [0, P]) and
 * BLK_EUNSUPPORTED (batch above 16).
 */
int blk_forward_chunks(const blk_config* cfg, const void* packed, int layer, int batch,
                       int tokens, int prefix, const int32_t* prefix_lens, const uint16_t* x,
                       const uint16_t* k_prefix, const uint16_t* v_prefix, int64_t prefix_stride,
                       uint16_t* y, uint16_t* k_new, uint16_t* v_new, int64_t new_stride, void* ws,
                       size_t* ws_bytes, void* stream);

/*
 * blk_forward_noalloc -- blk_forward without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, layouts, results and errors as blk_forward, minus ws and
 * ws_bytes.  The workspace is a static array inside the library, one copy per
 * GPU, 16 MiB (BLK_NOALLOC_SCRATCH_BYTES), held until the process ends; a
 * stage that needs more (its blk_forward size query) fails with BLK_ESIZE.
 * The first call on a device also enqueues a small kernel that zeroes the
 * array's synchronization region.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine) and records no operator timing.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (two streams, two threads) race and must be serialized by the
 * caller; one stream is fine.
 */
#define BLK_NOALLOC_SCRATCH_BYTES (16u << 20)
int blk_forward_noalloc(const blk_config* cfg, const void* packed, int layer, int batch,
                        int tokens, int prefix, const uint16_t* x, const uint16_t* k_prefix,
                        const uint16_t* v_prefix, int64_t prefix_stride, uint16_t* y,
                        uint16_t* k_new, uint16_t* v_new, int64_t new_stride, void* stream);

/*
 * prefix_prefill -- the prefix stage that builds the per-layer K/V caches a
 * denoise loop reads ([RT] §2: vision and language produce the KV cache once
 * per inference and the action expert reuses it over its denoise steps; §4.3:
 * when only the last layer's K/V is consumed, its attention and FFN are dead
 * work; §7.1: this stage runs on its own stream beside the loop).
 *
 * Runs layers 0..n_layers-1 of `packed` on the T = tokens prefix tokens x
 * (device bf16 [T][D], positions 0..T-1, no cached keys before them, no mask).
 * Layer l < n_layers - 1 is a full block stage whose output feeds layer l + 1;
 * every layer l writes its keys (after RoPE) and values to k_cache[l] and
 * v_cache[l] (host arrays of n_layers device pointers, each bf16 [T][Hkv][d],
 * 16-byte aligned); the last layer computes only its keys and values.
 * ws: device workspace (query with ws == NULL), zero-filled before first use.
 * Where a layer's attention leaves compute units free and its O + gate/up
 * weights reach 8 MiB, the attention launch carries extra workgroups that
 * read those weights ahead of their GEMMs (the weights of a chain of layers
 * stream from HBM).
 * Asynchronous on `stream`.  Errors: BLK_EINVAL, BLK_EUNSUPPORTED, BLK_ESIZE,
 * BLK_ESTATE, BLK_EHIP.
 */
int prefix_prefill(const blk_config* cfg, const void* packed, int n_layers, int tokens,
                   const uint16_t* x, uint16_t* const* k_cache, uint16_t* const* v_cache,
                   void* ws, size_t* ws_bytes, void* stream);

/*
 * flow_denoise -- the action expert's Euler flow-matching loop ([RT] §2-§4).
 *
 * For s = 0..n_steps-1: X = [state Ws + bs ; SiLU(a W1W2a + table[s]) W3 + b3]
 * ([N + 1][D]); X = block_l(X) for l = 0..n_layers-1 (layer l reads its own
 * prefix k_prefix[l], v_prefix[l], each device bf16 [P][Hkv][d]; chunk token t
 * at position P + t); v = RMSNorm(X[1:]) g_F W_out + b_out; a += dt_s v.
 *   k_prefix, v_prefix  host arrays of n_layers device pointers
 *   noise    device float32 [N][A]  a_0 (read only)
 *   state    device float32 [A]
 *   actions  device float32 [N][A]  a_{n_steps} (also the loop's running state)
 *   ws       device workspace (query with ws == NULL), zero-filled before first use
 * `packed` must hold a flow head prepared for exactly n_steps steps and at
 * least n_layers layers.  For layers whose O + gate/up weights reach 8 MiB
 * (and QKV weights 4 MiB), each attention launch carries extra workgroups that
 * read the layer's O and gate/up weights, and each down projection workgroups
 * that read the next layer's QKV weights, ahead of those launches (a stack of
 * layers streams its weights from HBM every step).  The whole loop is
 * captured once into a hipGraph keyed on (packed, n_layers, n_steps, P, every pointer argument); later calls
 * with the same key replay it with one launch, a changed key captures anew
 * (capture synchronizes the device once).  The key's buffers must stay valid
 * while the graph is cached (until blk_release or re-capture).
 * Errors: BLK_EINVAL, BLK_EUNSUPPORTED, BLK_ESIZE, BLK_ESTATE, BLK_EHIP.
 */
int flow_denoise(const blk_config* cfg, const void* packed, int n_layers, int n_steps,
                 int prefix, const uint16_t* const* k_prefix, const uint16_t* const* v_prefix,
                 const float* noise, const float* state, float* actions, void* ws,
                 size_t* ws_bytes, void* stream);

/* Message of the calling thread's last failed call ("" if none). */
const char* blk_last_error(void);

/* Destroys every cached graph and forgets every registered packed buffer.
 * Call with no library work in flight. */
void blk_release(void);

/* Library ABI version (bumped when a signature or a layout changes). */
int blk_version(void);

/*
 * blk_set_execution_mode -- how blk_forward and flow_denoise run a small chunk
 * (B*T <= 64 rows), process-wide:
 *   0 (default) automatic: the path this library version measures fastest
 *     for the shape (at present one kernel per operator everywhere);
 *   1 always one kernel per operator;
 *   2 the persistent stage kernel: one launch for the whole block or the whole
 *     denoise loop, its workgroups handing off through flags in the workspace
 *     ([TR]-style execution without launch gaps); BLK_EUNSUPPORTED where it
 *     does not cover the shape.
 * Results agree within rounding.  Large chunks (B*T > 64) always use
 * per-operator kernels.
 * Errors: BLK_EINVAL for another value.
 */
int blk_set_execution_mode(int mode);

/*
 * The persistent mode's workgroups wait for each other through memory: it
 * launches one workgroup per compute unit and assumes they are all resident at
 * once (nothing else may hold the GPU's compute units so that some of them
 * cannot start).  Every wait is bounded (about seconds): a wait that times out
 * sets the workspace's abort word (the 32-bit word at BLK_WS_ABORT_OFFSET),
 * every other wait then gives up, and the launch writes NaN over its outputs
 * (y, K_new and V_new, or the actions); later persistent launches on that
 * workspace do the same at once until the workspace is zero-filled again.
 * Since calls are asynchronous, such a call itself returns BLK_OK; the abort
 * is reported by:
 *
 * blk_workspace_status -- waits for `stream` (hipStreamSynchronize), then
 *   reads the abort word of device workspace `ws`: BLK_OK if clear,
 *   BLK_EABORTED if set (zero-fill the workspace to use it again).
 *   Errors: BLK_EINVAL (ws NULL), BLK_EHIP.
 */
int blk_workspace_status(const void* ws, void* stream);

/*
 * Operator timing.  The operators of one block stage, in order:
 */
#define BLK_OP_QKV 0        /* RMS(x), fused QKV GEMM, RoPE epilogue              */
#define BLK_OP_ATTENTION 1  /* chunk attention (and its key-slice merge)          */
#define BLK_OP_O_PROJ 2     /* O projection + residual                            */
#define BLK_OP_GATE_UP 3    /* RMS(h), gate/up GEMM, SiLU(gate) * up epilogue     */
#define BLK_OP_DOWN 4       /* down projection + residual                         */
#define BLK_OP_STAGE 5      /* the persistent stage kernel, as one operator       */
#define BLK_N_OPS 6

/*
 * blk_set_operator_timing -- enable (1) or disable (0) operator timing,
 * process-wide; either call discards what was accumulated.  While enabled,
 * every blk_forward call records a HIP event (created without the system-scope
 * fence, so no cache write-back is added) on its stream before its first
 * kernel and after each operator's last kernel (the work itself is unchanged),
 * so an operator's time is the interval between the event ahead of it and its
 * own.  At most 4096 calls are held between reads (BLK_ESIZE from blk_forward
 * beyond that); blk_forward on a stream under graph capture fails with
 * BLK_ESTATE while timing is on.  flow_denoise records nothing.
 * Errors: BLK_EINVAL for another value.
 */
int blk_set_operator_timing(int enable);

/*
 * blk_operator_times -- waits for the recorded events, adds their intervals
 * to per-operator totals and writes, for operator i < min(n, BLK_N_OPS),
 * avg_us[i] (host double, microseconds per call since timing was enabled) and
 * calls[i] (host int, timed calls; 0 with avg_us[i] = 0 for an operator that
 * never ran).  Errors: BLK_EINVAL (NULL arrays with n > 0, n < 0), BLK_EHIP.
 */
int blk_operator_times(double* avg_us, int* calls, int n);

/*
 * Measurement probes (not part of the block stage).  Benchmarks report their
 * results beside the chip's nominal peaks.  Both synchronize `stream` (they
 * time work on it with HIP events) and allocate no device memory.
 *
 * blk_probe_hbm_read -- sustained read bandwidth: `reps` passes of 16-byte
 *   non-temporal loads over the caller's device buffer `buf` (16-byte aligned,
 *   bytes >= 1 MiB and a multiple of 16; make it several times the 256 MB
 *   last-level cache so the passes come from HBM); *gb_per_s = bytes x reps /
 *   elapsed (1 GB = 1e9 bytes).
 * blk_probe_mfma_bf16 -- dense bf16 MFMA throughput: two waves per SIMD each
 *   run four independent chains of `iters` v_mfma_f32_32x32x16_bf16 on
 *   register operands; *tflops = 2 x 32 x 32 x 16 x MFMAs / elapsed, and
 *   *clock_ghz is the shader clock over one wave's loop (s_memtime cycles over
 *   the 100 MHz s_memrealtime counter).
 * Errors: BLK_EINVAL (NULL outputs, sizes out of range), BLK_EHIP; the message
 * is in blk_probe_last_error() (per calling thread).
 */
int blk_probe_hbm_read(const void* buf, size_t bytes, int reps, double* gb_per_s, void* stream);
int blk_probe_mfma_bf16(int iters, double* tflops, double* clock_ghz, void* stream);
const char* blk_probe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BLK_H_ */
