// kernels.h -- launch interface of the gfx950 kernels (internal to libqt).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qtk {

enum WType { W_F32 = 0, W_BF16 = 1, W_Q8 = 2, W_Q4 = 3 };
// block formats carry one fp16 scale per 32 weights along K; Q4 packs two
// 4-bit codes c per byte (even index in the low nibble), w = d * (c - 8)
__host__ __device__ constexpr bool w_blocked(int wt) { return wt == W_Q8 || wt == W_Q4; }
enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_GATED = 2 };

// Row r of a step belongs to slot  slot_base + r / rows_per_slot  and sits at
// position  pos_dev ? pos_dev[slot] : pos_base + r % rows_per_slot.
// Prompt chunks carry a device descriptor instead (pf, the PF_* words below):
// row r is row r % rows_per_slot of the chunk's stream i = r / rows_per_slot,
// slot pf[PF_SLOT + i], position pf[PF_R0] + r % rows_per_slot, and a padding
// row (not written to the ring) past the stream's pf[PF_LEN + i] rows;
// pos_base then only sizes the launch (the chunk's start on the host).
struct RowMap {
  int32_t slot_base;
  int32_t rows_per_slot;
  int32_t pos_base;
  const int32_t *pos_dev;
  const int32_t *pf = nullptr;
};

// Prompt-chunk descriptor words (int32; sampler words as in the decode's
// control block).  Up to PF_MAXROWS streams per chunk.
enum PfWord {
  PF_IDOFF = 0,  // first row of the chunk's ids in the staged id arrays
  PF_R0 = 1,     // position of the chunk's first row (every stream)
  PF_ITEMP = 2, PF_SEED_LO = 3, PF_SEED_HI = 4, PF_TOPK = 5,
  PF_SLOT = 8,   // [i] slot of stream i
  PF_LEN = 12,   // [i] prompt rows of stream i in the chunk (the rest is padding)
  PF_HEAD = 16,  // [i] chunk row of stream i's last prompt row, -1: its prompt goes on
  PF_T = 20,     // [i] stream i's prompt length
  PF_WORDS = 32
};
constexpr int PF_MAXROWS = 4;

struct Lin {
  const void *w;
  const uint16_t *sc;  // Q8 / Q4 block scales (fp16 bits), else null
};

// y[m][n] (epilogue) sum_k W[n][k] * x~[m][k]
//   x~ = act(x * rinv_m * gain)   when gain != null (RMSNorm prologue)
//   x~ = act(x)                   otherwise
struct GemvArgs {
  Lin seg[3];          // row segments (q|k|v) ...
  int32_t seg_end[3];  // ... rows [seg_end[i-1], seg_end[i]) read seg[i]
  int32_t nseg;
  Lin up;              // EPI_GATED: second matrix (u); seg[0] is the gate
  int32_t N, K;
  const float *x;
  int32_t x_stride;
  int32_t M;
  const void *gain;
  int32_t gain_bf16;
  float eps;
  int32_t act_bf16;
  float *y;
  int32_t y_stride;
  float *normed_out;   // block 0 stores x * rinv * gain (f32) here, stride K
  float *copy_out;     // EPI_RESID: also store the updated row here
  int32_t copy_stride;
};

struct QkArgs {
  const float *qkv;  // [M][(nq + 2 nkv) hd]
  int32_t M;
  RowMap rows;
  int32_t nq, nkv;
  const void *q_gain, *k_gain;
  int32_t gain_bf16;
  float eps;
  const float *rope_cos, *rope_sin;  // [rope_rows][hd/2]
  float *q_out;                      // [M][nq hd]
  void *ring_layer;                  // this layer's (slot 0, K) block
  int64_t slot_stride, kv_stride;    // elements
  int32_t P;                         // positions per (slot, layer, K|V, head)
  // Paged ring (page size 1): ptab[slot * P + pos] is the pool row of a
  // position, rows_per_head the pool's rows; null: the dense ring (row = pos)
  const int32_t *ptab;
  int32_t rows_per_head;
};

struct AttnArgs {
  const float *q;  // [M][nq hd]
  int32_t M;
  RowMap rows;
  int32_t nq, nkv;
  const void *ring_layer;
  int64_t slot_stride, kv_stride;
  int32_t P;
  const int32_t *ptab;    // paged ring: pool row of (slot, position) at [slot * P + pos], or null
  int32_t rows_per_head;  // rows of one (layer, K|V, head): P (dense) or the pool's
  int32_t tile;       // positions per tile (fixed absolute boundaries)
  int32_t max_tiles;  // tiles per row in the partial buffer
  int32_t grid_tiles; // grid z: tiles launched (rows' positions known to stay below grid_tiles * tile), or 0: max_tiles
  float scale;
  float *o;           // [M][nq hd]
  float *part;        // [M][nq][max_tiles][hd + 2]
  // Fused q/k norm + RoPE + set_rows (rows_per_slot <= 2): q is built from
  // qkv instead of read from q, and the K/V rows of the step's new positions
  // are built in the workgroup and written to the ring by the row they
  // belong to.  qkv null: q holds the rotated queries and the ring the rows.
  const float *qkv;   // [M][(nq + 2 nkv) hd]
  const void *q_gain, *k_gain;
  int32_t gain_bf16;
  float eps;
  const float *rope_cos, *rope_sin;  // [rope_rows][hd/2]
};

struct GatherArgs {
  const void *code_emb, *text_emb;
  int32_t tab_bf16, H, Vc, G;
  const int32_t *codes;  // row r: codes[r * codes_stride + g]; null: text rows only
  int32_t codes_stride;
  const int32_t *text;   // row r: text[r * text_stride]
  int32_t text_stride;
  const int32_t *ctl;    // if set, codes/text advance by ctl[0] * frame_stride_*
  int32_t frame_stride_codes, frame_stride_text;
  float *x;
  int32_t M;
  float *x0_dump;
  int32_t *gather_dump;  // [M][G+1]
  float *ssq;            // optional: row sums of squares in 32-column slots [M][H/32]
};

struct PredInArgs {
  const float *bridge;
  const void *code_emb;
  int32_t tab_bf16, H, G, B;
  const int32_t *c0_state;
  const int32_t *ctl;  // [0] frame index base, [1] forcing
  int32_t k;           // frame within the replay
  int32_t *cin, *cout; // [frames][B][G]
  float *x;            // rows 2b = bridge[b], 2b+1 = E_0[c0]
  float *ssq;          // optional: row sums of squares in 32-column slots [2B][H/32]
};

enum ArgMode { AM_PRED = 0, AM_TALKER = 1, AM_PREFILL = 2 };

struct ArgmaxArgs {
  const float *logits;
  int32_t Vc, M, mode;
  int32_t j;  // AM_PRED: head index (code j+1)
  const int32_t *ctl;
  int32_t k, B, G;
  int32_t *cin, *cout;
  int32_t *c0_state, *pos, *tpos_dump;
  const void *code_emb;
  int32_t tab_bf16, H;
  float *x_next;  // AM_PRED: row b <- E_{j+1}[code] when j+1 < G-1
  float *ssq;     // optional: x_next row sums of squares in 32-column slots [M][H/32]
  // AM_PREFILL: row r is stream r of a prompt chunk (ctl = its descriptor,
  // PF_* words); a stream whose prompt ends in the chunk (PF_HEAD >= 0) gets
  // c0, pos = its prompt length, its bridge row (bridge_src row r) and its
  // logits row (logits_out row slot)
  const float *bridge_src;
  float *bridge, *logits_out;
  // Sampling (sampler.h), read from the control words: ctl[2] = float bits
  // of 1/T (0: greedy), ctl[3], ctl[4] = seed low, high, ctl[5] = top_k (0:
  // all; needs Vc <= 2048); q = the prompt length for AM_PREFILL.
};

// Batched projection on MFMA: y = epi(act(norm(x)) . W^T) for M <= GEMM_MAX_ROWS rows (64-row blocks),
// bf16, q8 or q4 weights with bf16 operands.  Tiles of 32 output columns (gated:
// 32 gate + 32 up rows) x 64 rows x kpw consecutive 256-wide K slices per
// workgroup; the last workgroup of a tile to finish sums the workgroups'
// partials in order and applies the epilogue.
constexpr int GEMM_MAX_ROWS = 512;
struct GemmArgs {
  Lin seg[3];          // row segments (q|k|v) ...
  int32_t seg_end[3];  // ... rows [seg_end[i-1], seg_end[i]) read seg[i]
  int32_t nseg;
  Lin up;              // EPI_GATED: the up matrix (seg[0] is the gate)
  int32_t N, K, M;
  const float *x;
  int32_t x_stride;
  const void *gain;    // RMSNorm gain, or null: no norm
  int32_t gain_bf16;
  float eps;
  const float *ssq;    // with gain: row m's sums of squares at ssq[m * ssq_stride + i], i < K / 32
  int32_t ssq_stride;
  float *y;
  int32_t y_stride;
  float *ssq_out;      // EPI_RESID: new rows' sums of squares in 32-column slots [M][N/32]
  float *normed_out;   // optional: f32 normed rows [M][K] (the talker bridge)
  float *copy_out;     // EPI_RESID: also store the new row here
  int32_t copy_stride;
  float *part;         // [K/256][M][N or 2N] split-K partials
  uint32_t *cnt;       // [tiles] arrival counters, zero between launches
  int32_t kpw;         // 256-wide K slices per workgroup (0 or 1, or 2 where it divides K/256)
};
hipError_t launch_gemm(int wtype, int epi, const GemmArgs &a, hipStream_t s);

// Prompt chunks: row PF_HEAD[i] of x (or row 0 when negative) -> row i of xh,
// for the chunk's n streams: the last row of each prompt that ends in the
// chunk, whose final-norm output is the bridge and whose head logits decide
// frame 0's first code ([QT-log] per-layer K/V ring entry: a T-row prefill,
// then one row per decode step).
hipError_t launch_pf_rows(const int32_t *pf, const float *x, float *xh, int32_t n, int32_t H, hipStream_t s);

hipError_t launch_gemv(int wtype, int epi, const GemvArgs &a, hipStream_t s);
hipError_t launch_qk_rope_kv(int hd, int kv_bf16, const QkArgs &a, hipStream_t s);
// Causal attention of a prompt chunk (a.rows.pf set; hd 128, bf16 K/V, GQA
// group 1, 2 or 4; else hipErrorInvalidValue): 16 query positions x one KV
// head's query heads per workgroup, MFMA with f32 operands, output in a.o.
hipError_t launch_attn_prompt(int hd, int kv_bf16, const AttnArgs &a, int n_streams, hipStream_t s);
hipError_t launch_attention(int hd, int kv_bf16, const AttnArgs &a, bool combine, hipStream_t s);
hipError_t launch_gather(const GatherArgs &a, hipStream_t s);
hipError_t launch_pred_input(const PredInArgs &a, hipStream_t s);
hipError_t launch_argmax(const ArgmaxArgs &a, hipStream_t s);
hipError_t launch_advance(int32_t *ctl, int32_t K, hipStream_t s);
// streaming read of `bytes` (a multiple of 16) at src; writes kStreamGrid *
// 256 words to sink
constexpr int kStreamGrid = 2048;
hipError_t launch_stream_read(const void *src, size_t bytes, void *sink, hipStream_t s);

}  // namespace qtk
