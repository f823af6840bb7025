/*
 * qt.h -- C ABI of the MI355X (gfx950) per-frame decode library.
 *
 * One codec frame = one talker step + 15 code-predictor micro-steps, decoded
 * greedily (or by temperature sampling, qt_set_sampler) on one GPU.  All compute runs in the library's HIP kernels; the
 * caller supplies device memory (weights, the K/V ring, a scratch arena) and a
 * HIP stream, typically from PyTorch.  No entry point allocates device memory.
 *
 * Sources (page title, section):
 *   [QT-log]   qwentts.cpp, commit log of src/pipeline-tts.h
 *   [QT-tests] qwentts.cpp, commit log of the tests branch
 *   [MC-opt]   MiniCPM-o 4.5 single-GPU engine, docs/optimizations.md
 *
 * Conventions
 *   - Every entry point returns int32_t status: QT_OK (0) or a negative QT_E_*.
 *     A failing call changes no state: arguments are validated on the host
 *     before any launch.  The one exception is QT_E_HIP from a call that had
 *     already launched work (a HIP runtime failure, or a timed-out wait of
 *     the persistent kernel): the slots that call was decoding may hold
 *     partial results, so they are marked un-prefilled and the next
 *     qt_decode_frame returns QT_E_STATE until qt_prefill or
 *     qt_set_slot_state restores them.  No failure is silent: an empty or
 *     partial result always comes with an error status ([QT-log], clone-mode
 *     entry: an encoder pass that returned empty without an error).
 *     qt_last_error() describes the last failure.
 *   - "device" pointers are HIP device addresses; "host" pointers are ordinary
 *     host memory, read or written only during the call.  The library keeps
 *     device pointers it is given for the lifetime of the context; the caller
 *     keeps that memory alive and at a fixed address until qt_free().
 *   - Matrices are row-major [out][in]; "bf16" means IEEE bfloat16 bits.
 *   - One context is driven by one host thread.
 */
#ifndef QT_H
#define QT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Closed ABI range: a caller built against any version in
   [QT_ABI_MIN_VERSION, QT_ABI_VERSION] is accepted; both bounds are checked
   ([QT-tests], codec left context / ABI range entry: the range check rejects
   a version past either bound). */
#define QT_ABI_MIN_VERSION 1
#define QT_ABI_VERSION 5 /* 2: qt_set_sampler; 3: qt_stream_read; 4: paged ring (QT_F_PAGED); 5: qt_prefill_rows */

#define QT_OK 0
#define QT_E_ABI (-1)          /* abi_version outside the closed range (checked first) */
#define QT_E_ARG (-2)          /* bad argument: NULL, negative count, bad flag, struct_size */
#define QT_E_SIZE (-3)         /* ring or arena smaller than qt_query_sizes() */
#define QT_E_RANGE (-4)        /* a code id >= codebook_size or text id >= text_rows */
#define QT_E_STATE (-5)        /* slot not prefilled, or dump read without QT_F_DUMP */
#define QT_E_CONTEXT_FULL (-6) /* the talker ring cannot hold the requested positions */
#define QT_E_HIP (-7)          /* a HIP runtime call failed */
#define QT_E_UNSUPPORTED (-8)  /* shape outside what the kernels implement */

/* storage of linear (projection and head) weights */
#define QT_LIN_F32 0
#define QT_LIN_BF16 1
#define QT_LIN_Q8 2 /* int8 values [N][K] + fp16 scale per 32 along K: [N][K/32] */
/* 4-bit blocks of this library's own definition (the qwentts.cpp commit log's
   TTFA table lists a 4-bit column but defines no block): uint8 [N][K/2], weight
   k in byte k/2, low nibble for even k, code c in 0..15 standing for c - 8; fp16
   scale d per 32 along K: [N][K/32]; w = d * (c - 8).  Decoded by both paths,
   like QT_LIN_Q8. */
#define QT_LIN_Q4 3

/* context flags */
#define QT_F_DUMP 1u  /* keep per-step readbacks (logits, bridge, gather ids, hidden) */
#define QT_F_EAGER 2u /* launch kernels directly instead of replaying a hipGraph */
#define QT_F_OPS 4u   /* one kernel per op (hipGraph) even where the persistent
                         frame kernel applies (single stream); for comparisons */
#define QT_F_TRACE 8u /* persistent kernel: workgroup 0 stamps every phase of the
                         first frame of a call (read with QT_DUMP_TRACE) */
#define QT_F_PAGED 16u /* paged talker ring, page size 1 ([MC-opt] core table:
                          paged KV for many streams): one pool of pool_rows
                          rows per (layer, K|V, head) shared by every slot,
                          rows handed out as positions are first written and
                          returned when a slot is prefilled again; the page
                          table (slot, position) -> row is device data, so the
                          graph never changes.  Decodes on the per-op path. */

typedef struct qt_model_desc {
  int32_t hidden;              /* H: width of talker and predictor */
  int32_t n_q_heads;           /* nq */
  int32_t n_kv_heads;          /* nkv (divides nq) */
  int32_t head_dim;            /* hd: 64 or 128 */
  int32_t ffn;                 /* F: SiLU-multiply width */
  int32_t talker_layers;       /* Lt */
  int32_t predictor_layers;    /* Lp */
  int32_t codebooks;           /* G: codes per frame (16) */
  int32_t codebook_size;       /* Vc: entries per codebook = width of every head */
  int32_t text_rows;           /* Vt: rows of the text / pad overlay table */
  int32_t talker_positions;    /* P: talker ring positions (multiple of 256) */
  int32_t predictor_positions; /* Q: predictor cache positions (== G) */
  int32_t lin_type;            /* QT_LIN_* */
  int32_t tab_bf16;            /* code / text tables and norm gains: 1 bf16, 0 f32 */
  int32_t kv_bf16;             /* ring rows: 1 bf16, 0 f32 */
  int32_t act_bf16;            /* 1: matmul activation operands rounded to bf16 (RNE) */
  double eps;                  /* RMSNorm epsilon */
  double rope_theta;           /* RoPE base */
} qt_model_desc;

typedef struct qt_linear {
  const void *w;      /* device: f32 / bf16 [N][K], int8 [N][K] (QT_LIN_Q8) or uint8 [N][K/2] (QT_LIN_Q4) */
  const void *scales; /* device: QT_LIN_Q8 / QT_LIN_Q4 only, fp16 bits [N][K/32]; else NULL */
} qt_linear;

/* One decoder layer (pre-norm; [MC-opt] core table: residual add + RMSNorm,
   q/k norm + RoPE, SiLU-multiply).  Norm gains are [H] or [hd]. */
typedef struct qt_layer_weights {
  const void *attn_norm; /* [H] */
  qt_linear wq;          /* [nq*hd][H] */
  qt_linear wk;          /* [nkv*hd][H] */
  qt_linear wv;          /* [nkv*hd][H] */
  const void *q_norm;    /* [hd], shared by all query heads */
  const void *k_norm;    /* [hd], shared by all key heads */
  qt_linear wo;          /* [H][nq*hd] */
  const void *mlp_norm;  /* [H] */
  qt_linear wg;          /* [F][H] gate */
  qt_linear wu;          /* [F][H] up */
  qt_linear wd;          /* [H][F] down */
} qt_layer_weights;

typedef struct qt_weights {
  const void *code_emb;                /* device [G][Vc][H]: table g feeds code g
                                          ([QT-log] AR inputs entry) */
  const void *text_emb;                /* device [Vt][H]: text / pad overlay rows */
  const qt_layer_weights *talker;      /* host array [Lt], read during qt_init */
  const void *talker_norm;             /* device [H] */
  qt_linear talker_head;               /* [Vc][H] */
  const qt_layer_weights *predictor;   /* host array [Lp], read during qt_init */
  const void *predictor_norm;          /* device [H] */
  const qt_linear *predictor_heads;    /* host array [G-1], each [Vc][H] */
} qt_weights;

/* Everything a context is built from, read once by qt_init ([QT-tests],
   codec left context / ABI range entry: an init-params struct resolved once
   at load, versioned by the closed ABI range above). */
typedef struct qt_init_params {
  uint32_t abi_version; /* QT_ABI_VERSION of the caller's header */
  uint32_t struct_size; /* sizeof(qt_init_params) */
  qt_model_desc model;
  qt_weights weights;
  /* Caller-owned device memory, 256-byte aligned, >= qt_query_sizes():
     ring  = talker ring [B][Lt][2][nkv][P][hd] then predictor cache
             [B][Lp][2][nkv][Q][hd] ([2] = K, V), element bf16 or f32 per
             kv_bf16 ([QT-log] per-layer K/V ring entry).  Row `pos` of a
             (slot, layer, K|V, head) holds that position's vector.
     arena = the library's fixed-address scratch (state, activations, io). */
  void *ring;
  size_t ring_bytes;
  void *arena;
  size_t arena_bytes;
  int32_t max_batch;           /* B: streams decoded together (slots 0..B-1) */
  int32_t frames_per_replay;   /* K: frames per graph replay (a call's tail replays a 1-frame graph) */
  int32_t max_frames_per_call; /* frames staged per upload; longer calls loop */
  uint32_t flags;              /* QT_F_* */
  void *stream;                /* hipStream_t, caller-owned; non-default unless QT_F_EAGER */
  /* ABI 4: with QT_F_PAGED, the talker ring's rows per (layer, K|V, head),
     shared by all slots (>= 1); the ring is then the pool
     [Lt][2][nkv][pool_rows][hd] followed by the predictor cache
     [B][Lp][2][nkv][Q][hd], sized by qt_query_paged_ring.  Callers of an
     older ABI pass the structure without this field (struct_size up to
     `stream`): a dense ring. */
  int32_t pool_rows;
} qt_init_params;

typedef struct qt_ctx qt_ctx;

/* ABI version of the loaded library (the library's own query). */
int32_t qt_abi_version(void);

/* Pure host computation of the device memory a context needs (the
   library's own helper: the ring is sized once for P positions, as the
   [QT-log] per-layer K/V ring entry sizes its buffer at init for the
   longest sequence; the arena holds the fixed-address buffers of the
   [QT-log] persistent-arena entry).
   ring_bytes = B*Lt*2*nkv*P*hd*e + B*Lp*2*nkv*Q*hd*e with e = 2 (bf16) or 4.
   Errors: QT_E_ARG (NULL outputs, non-positive sizes), QT_E_UNSUPPORTED. */
int32_t qt_query_sizes(const qt_model_desc *model, int32_t max_batch, int32_t frames_per_replay,
                       int32_t max_frames_per_call, uint32_t flags, size_t *ring_bytes,
                       size_t *arena_bytes);

/* Ring bytes of a QT_F_PAGED context (the library's own helper; the arena is
   the same as qt_query_sizes gives): talker pool Lt*2*nkv*pool_rows*hd*e plus
   the predictor cache B*Lp*2*nkv*Q*hd*e.  A pool holding every slot's
   longest context is the dense ring's size at most; ragged contexts need
   their sum.  Errors: QT_E_ARG (NULL output, non-positive sizes),
   QT_E_UNSUPPORTED. */
int32_t qt_query_paged_ring(const qt_model_desc *model, int32_t max_batch, int32_t pool_rows, size_t *ring_bytes);

/* Validates, binds caller memory, uploads the RoPE table, and (unless
   QT_F_EAGER) captures the K-frame graph on params->stream.  Everything a
   context needs is fixed here, once, from qt_init_params ([QT-tests], codec
   left context / ABI range entry: settings move into the init params and
   are resolved once at load); every later call reuses the same device
   addresses ([QT-log], persistent-arena entry: fixed tensor addresses let a
   captured graph replay without an update).  All slots start un-prefilled.
   The persistent frame kernel is chosen only where every one of its
   workgroups fits on the device at once (one per compute unit, checked with
   the occupancy query); it is launched cooperatively, so the runtime either
   makes them all resident together or refuses the launch.
   Errors: QT_E_ABI first, then QT_E_ARG, QT_E_UNSUPPORTED, QT_E_SIZE,
   QT_E_HIP.  *out is set only on success. */
int32_t qt_init(const qt_init_params *params, qt_ctx **out);

/* Prefill of one slot with T prompt rows ([QT-log] per-layer K/V ring entry:
   prefill resets the cache and writes T positions).  Row p's input is
   sum_g code_emb[g][codes[p][g]] + text_emb[text_ids[p]] (codes may be NULL:
   text rows only).  Writes ring rows [0, T), sets the slot's bridge (final
   normed hidden of row T-1), c0 (argmax of the talker head) and pos = T.
   codes: host [T][G] or NULL; text_ids: host [T].  Synchronous.  Paged ring:
   the slot's rows go back to the pool first, then it takes T rows.  The
   same as qt_prefill_rows with one stream.
   Errors: QT_E_ARG, QT_E_RANGE, QT_E_CONTEXT_FULL (T > P, or a paged pool
   without T free rows), QT_E_HIP. */
int32_t qt_prefill(qt_ctx *ctx, int32_t slot, int32_t T, const int32_t *codes,
                   const int32_t *text_ids);

/* Prefill of n streams (1 <= n <= 4) in one call, each as qt_prefill would
   ([MC-opt] round-18 table, talker chunk-prefill graphs: graphs per row count
   1-4 and token bucket, first codes decided in the same call).  The prompts
   run in chunks: a chunk holds the same positions [r0, r0 + t) of every
   stream whose prompt is not yet done, t a token bucket (a power of two from
   16 to 512, at most 512 rows per chunk; the ring's last positions may make
   the final chunk shorter); a shorter prompt's rows past its end are padding, which
   writes no ring row and changes no result, so each slot ends exactly as
   after qt_prefill of its own prompt (bit for bit).  Unless QT_F_EAGER,
   every chunk replays a graph captured once per (streams, t, attention
   tiles, codes given, last chunk of some prompt) on the context's stream
   and kept until qt_free; the first call of a new shape captures it (a
   context keeps up to 128 such graphs; chunks of further shapes launch their
   kernels directly, with the same results).
   slots: host [n], distinct; lengths: host [n], each in [1, P]; codes: host
   [sum(lengths)][G] (stream i's rows after streams 0..i-1's) or NULL (text
   rows only, for every stream); text_ids: host [sum(lengths)], same order.
   Synchronous.  Paged ring: the slots' rows go back to the pool first, then
   each takes its prompt's rows.
   Errors: QT_E_ARG (n outside [1, 4], NULLs, a slot outside [0, B) or given
   twice, a length <= 0), QT_E_RANGE, QT_E_CONTEXT_FULL (a length > P, or a
   paged pool without the rows), QT_E_HIP; every check is made before the
   first launch, and after a QT_E_HIP the slots are un-prefilled. */
int32_t qt_prefill_rows(qt_ctx *ctx, int32_t n, const int32_t *slots, const int32_t *lengths,
                        const int32_t *codes, const int32_t *text_ids);

/* Decodes n_frames frames for all B slots.  With one slot (B = 1) and a shape
   the persistent kernel implements, one kernel launch runs every phase of the
   frames (qt_path() reports which path a context uses); otherwise each K-frame
   block is one replay of a graph of per-op kernels, and the frames past the
   call's last whole block replay a second, 1-frame graph (adaptive K: a short
   call, such as a stream's first frame, is not held to K frames, while long
   calls keep K-frame replays; [MC-opt] experiments table: K trades
   throughput against time to first audio).  Any n_frames > 0.
   overlay_ids: host [n][B] (frame f's talker step adds text_emb row
   overlay_ids[f][b]).  codes_out: host [n][B][G]: codes_out[f][b][0] is the
   talker's greedy code for frame f, [1..G-1] the predictor's.  forced_codes:
   NULL, or host [n][B][G] teacher-forcing codes that are fed back instead of
   the argmax results (codes_out still receives every argmax).  Synchronous:
   codes are in codes_out on return.  Only ids cross the host boundary per
   frame ([QT-log] set_rows / hot-loop entry).
   With a sampler set (qt_set_sampler) codes_out holds the sampled codes.
   Errors: QT_E_ARG (n_frames <= 0, NULLs), QT_E_RANGE, QT_E_STATE (a slot not
   prefilled), QT_E_CONTEXT_FULL (pos + n_frames > P, or a paged pool
   without the rows the new positions need; checked before any launch),
   QT_E_HIP. */
int32_t qt_decode_frame(qt_ctx *ctx, int32_t n_frames, const int32_t *overlay_ids,
                        int32_t *codes_out, const int32_t *forced_codes);

/* For callers that cannot allocate device memory (code that must not call
   hipMalloc: tight serving loops, harnesses that forbid allocation): the same
   decode as qt_decode_frame, with the same arguments, results and errors,
   but the persistent kernel's scratch -- its tagged exchange words and its
   error flag -- lives in a static device array of the library (512 KiB, one
   per device, held until the process ends) instead of the context's arena.
   The call allocates nothing: it clears the used part of that array on the
   context's stream (other contexts' calls leave their tags there), launches,
   and copies the codes back through the pinned staging that qt_init made.
   Every context on a device shares that device's array: calls that overlap
   on one device race and must be serialised by the caller.
   Errors: those of qt_decode_frame; QT_E_UNSUPPORTED if the context does not
   decode on the persistent kernel (qt_path() != QT_PATH_FRAME); QT_E_SIZE if
   the model's exchange region exceeds 512 KiB (the 28-layer, 1,024-wide
   model with a 4,096-position ring needs 452 KiB; 8 KV heads with rings of
   5,632 positions or more exceed it). */
int32_t qt_decode_frame_noalloc(qt_ctx *ctx, int32_t n_frames, const int32_t *overlay_ids,
                                int32_t *codes_out, const int32_t *forced_codes);

/* Snapshot / restore of a slot's non-ring state (the library's own calls,
   used to restart a decode from a saved or injected state): next talker
   position, the pending code 0, and the bridge (host float [H]; the bridge
   is the [QT-log] set_rows entry's device-resident talker hidden).  The
   ring itself is caller memory at the documented layout.  set marks the slot
   prefilled.  Paged ring: set needs rows for positions [0, pos) already
   given to the slot (by its prefill and decodes).
   Errors: QT_E_ARG, QT_E_RANGE (pos outside [1, P], c0 outside [0, Vc)),
   QT_E_STATE (paged: the slot holds fewer than pos rows). */
int32_t qt_get_slot_state(qt_ctx *ctx, int32_t slot, int32_t *pos, int32_t *c0, float *bridge);
int32_t qt_set_slot_state(qt_ctx *ctx, int32_t slot, int32_t pos, int32_t c0,
                          const float *bridge);

/* Readbacks of the last decoded frame (QT_F_DUMP only; host readbacks of
   hidden state exist only in this mode, as in [QT-log] set_rows entry).
   kind and host layout:
     QT_DUMP_TALKER_LOGITS f32 [B][Vc]       (after qt_prefill: its last row)
     QT_DUMP_PRED_LOGITS   f32 [G-1][B][Vc]
     QT_DUMP_BRIDGE        f32 [B][H]
     QT_DUMP_X0            f32 [B][H]        talker input gather-sum
     QT_DUMP_GATHER        i32 [B][G+1]      codes fed to the gather, overlay id
     QT_DUMP_TPOS          i32 [B]           talker K/V write position
     QT_DUMP_HIDDEN        f32 [Lt][B][H]    talker residual after each layer
     QT_DUMP_TRACE         u64 [1024][8]     QT_F_TRACE only: rows 0..767 per GEMV phase of the
                                             first GEMV workgroup (kind | stack << 8 | layer << 16 |
                                             step << 24, start, inputs in, end, norm done, GEMV done,
                                             the first wave's poll done, the weight slice landed); rows
                                             768.. per attention event of workgroup 0 (kind word,
                                             start, inputs in, end).  Wall-clock stamps are 100 MHz
                                             ticks; kind 255 ends each part
   bytes must equal the kind's size.  Errors: QT_E_STATE, QT_E_ARG, QT_E_HIP. */
#define QT_DUMP_TALKER_LOGITS 1
#define QT_DUMP_PRED_LOGITS 2
#define QT_DUMP_BRIDGE 3
#define QT_DUMP_X0 4
#define QT_DUMP_GATHER 5
#define QT_DUMP_TPOS 6
#define QT_DUMP_HIDDEN 7
#define QT_DUMP_TRACE 8
int32_t qt_read_dump(qt_ctx *ctx, int32_t kind, void *host_dst, size_t bytes);

/* Measurement hook (the library's own): launches one kernel of the frame
   `reps` times, in the
   launch configuration the frame uses at batch B, between two HIP events on
   the context's stream, and reports the average duration per launch
   (microseconds) and the algorithmic bytes one launch moves (weights once,
   activations in and out).  Successive launches walk every layer's weights
   (talker then predictor), as the frame does, so no launch finds its weights
   in a cache a previous launch filled.  Writes only arena scratch; the slots'
   state is untouched.  Synchronous.
     QT_KERNEL_GEMV_GATE_UP   RMSNorm + gate/up projection + SiLU-multiply (the
                              largest weight stream of a layer) as the per-op
                              decode path runs it for the context's batch: the
                              split-K MFMA GEMM for 1..512 rows with bf16, q8 or
                              q4 weights, the GEMV for f32 weights or widths the
                              GEMM does not take
   Errors: QT_E_ARG, QT_E_HIP, QT_E_UNSUPPORTED. */
#define QT_KERNEL_GEMV_GATE_UP 1
int32_t qt_time_kernel(qt_ctx *ctx, int32_t kernel, int32_t reps, double *avg_us,
                       double *bytes_per_launch);

/* Sampler of every later qt_prefill / qt_decode_frame call of ctx (the pages
   keep the sampler inside the decode graph: [QT-tests] fused codec mode removed
   entry; the distribution is this library's definition).  temperature 0 (the
   default) is the greedy argmax.  temperature T > 0: each code is
   argmax_n (l_n * (1/T) + g_n), lowest index on ties, over its head's f32
   logits l; 1/T is rounded to float once, the product and sum are float
   operations, g_n = -log(-log(u_n)) (double, rounded to float once) with
   u_n = ((x >> 11) + 0.5) * 2^-53 and x the first word of Philox4x64-10
   (Salmon et al., SC'11) at counter (n, j, q, slot), key (seed, 0); j is the
   code's index in its frame (0: the talker's), q the frame's talker position
   (a talker head at position p decides frame p + 1; qt_prefill of T rows
   decides frame T), slot the stream.  This draws each code from
   softmax(l / T).  top_k > 0: only the top_k largest logits compete (the draw
   is from softmax(l / T) restricted to them); equal logits at the boundary
   rank by lower index, as in the argmax.  top_k = 0 (or >= codebook_size):
   every logit.  Host only: no GPU call, no graph recapture.
   Every decode path implements it (on the persistent kernel every
   workgroup polls the head's logits and makes the same pick).
   Errors: QT_E_ARG (NULL ctx, temperature negative, NaN or infinite, top_k
   negative), QT_E_UNSUPPORTED (top-k with codebook_size > 2048). */
int32_t qt_set_sampler(qt_ctx *ctx, float temperature, int32_t top_k, uint64_t seed);

/* Measurement hook (the library's own): the achievable HBM read bandwidth
   that the decode kernels are compared with.  Reads `bytes` at src (device,
   16-byte aligned, a multiple of 16 and at least 1 MiB; pass well above the
   256 MB last-level cache for an HBM figure) with a plain streaming-read
   kernel, once untimed and then `reps` times between two HIP events on
   `stream` (hipStream_t; NULL: the default stream), and reports the average
   duration per pass in microseconds.  sink: device scratch of sink_bytes >=
   2 MiB that the kernel overwrites.  Synchronous.  Needs no context.
   Errors: QT_E_ARG, QT_E_SIZE (sink too small), QT_E_HIP. */
int32_t qt_stream_read(const void *src, size_t bytes, void *sink, size_t sink_bytes, int32_t reps, void *stream,
                       double *avg_us);

/* Decode path of a context (the library's own query): QT_PATH_FRAME
   (persistent frame kernel),
   QT_PATH_GRAPH (per-op kernels replayed as a hipGraph) or QT_PATH_EAGER. */
#define QT_PATH_FRAME 1
#define QT_PATH_GRAPH 2
#define QT_PATH_EAGER 3
int32_t qt_path(const qt_ctx *ctx);

/* Destroys graphs and host state; never frees caller memory (the caller
   owns it, as in the [QT-log] clone-mode entry the caller holds its buffers
   until the library returns).  NULL is a no-op. */
void qt_free(qt_ctx *ctx);

/* Last error text of ctx (of the calling thread when ctx is NULL): every
   failure carries one ([QT-log], clone-mode entry: no silent failures). */
const char *qt_last_error(const qt_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif /* QT_H */
