// api.cpp -- host side of libqt: validation, arena layout, frame schedule,
// hipGraph capture/replay and the C entry points declared in include/qt.h.
//
// Sources (page title, section):
//   [QT-log]   qwentts.cpp, commit log of src/pipeline-tts.h
//   [QT-tests] qwentts.cpp, commit log of the tests branch
//   [MC-opt]   MiniCPM-o 4.5 single-GPU engine, docs/optimizations.md
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "../../include/qt.h"
#include "frame.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

constexpr int kPrefillChunk = 512;  // prompt rows per prefill step (at most qtk::GEMM_MAX_ROWS)
constexpr int kPfMinRows = 16;      // smallest token bucket of a prompt chunk
constexpr size_t kPfMaxGraphs = 128; // prompt-chunk graphs a context keeps (further shapes launch eagerly)
constexpr int kPfSlicesPerWg = 2;   // 256-wide K slices per GEMM workgroup in prompt chunks
constexpr int kTile = 256;         // talker attention tile (window padding unit)
constexpr size_t kAlign = 256;
constexpr int kMaxWG = 1024;       // workgroups of the persistent kernel (>= CUs)
constexpr int kXchRep = 1;         // copies of the frame kernel's broadcast rows (1-8 measured alike)

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Byte offsets of every arena buffer; a pure function of the shapes.
struct Layout {
  size_t rope_cos, rope_sin, pos, c0, bridge, ctl, overlay, cin, cout;
  size_t x, qkv, q, part, o, z, logits_t, logits_p;
  size_t ptab;  // paged ring: pool row of (slot, position), int32 [B][P]
  size_t ssq, gpart, gcnt;  // batched projections: row sums of squares, split-K partials, tile counters
  size_t gcnt_bytes;
  size_t x0_dump, hidden_dump, gather_dump, tpos_dump, pf_codes, pf_text;
  size_t pf_desc, pf_xh, pf_lg, pf_br;  // prompt chunks: descriptor, head rows, logits, bridge rows
  // persistent frame kernel: weight tables, tagged exchange words, error flag
  size_t f_tl, f_pl, f_heads, f_heads_sc, f_xq, f_qkv, f_o, f_z, f_amax, f_lgx, f_part, f_err, f_trace;
  size_t xch_words;  // words between copies of the exchange rows
  size_t f_xch_begin;
  size_t total;
  int32_t rows;       // activation rows held
  int32_t max_tiles;  // talker attention tiles
};

struct Dims {
  int32_t H, nq, nkv, hd, F, Lt, Lp, G, Vc, Vt, P, Q, qd, kd, nqkv;
};

Dims dims_of(const qt_model_desc &m) {
  Dims d;
  d.H = m.hidden; d.nq = m.n_q_heads; d.nkv = m.n_kv_heads; d.hd = m.head_dim; d.F = m.ffn;
  d.Lt = m.talker_layers; d.Lp = m.predictor_layers; d.G = m.codebooks; d.Vc = m.codebook_size;
  d.Vt = m.text_rows; d.P = m.talker_positions; d.Q = m.predictor_positions;
  d.qd = d.nq * d.hd; d.kd = d.nkv * d.hd; d.nqkv = d.qd + 2 * d.kd;
  return d;
}

Layout layout_of(const Dims &d, int32_t B, int32_t maxF) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  L.rows = 2 * B > kPrefillChunk ? 2 * B : kPrefillChunk;
  L.max_tiles = d.P / kTile;
  const size_t R = (size_t)L.rows;
  L.rope_cos = take(sizeof(float) * d.P * (d.hd / 2));
  L.rope_sin = take(sizeof(float) * d.P * (d.hd / 2));
  L.pos = take(sizeof(int32_t) * B);
  L.c0 = take(sizeof(int32_t) * B);
  L.bridge = take(sizeof(float) * B * d.H);
  L.ctl = take(64);
  L.overlay = take(sizeof(int32_t) * (size_t)maxF * B);
  L.cin = take(sizeof(int32_t) * (size_t)maxF * B * d.G);
  L.cout = take(sizeof(int32_t) * (size_t)maxF * B * d.G);
  L.x = take(sizeof(float) * R * d.H);
  L.qkv = take(sizeof(float) * R * d.nqkv);
  L.q = take(sizeof(float) * R * d.qd);
  L.part = take(sizeof(float) * R * d.nq * L.max_tiles * (d.hd + 2));
  L.o = take(sizeof(float) * R * d.qd);
  L.z = take(sizeof(float) * R * d.F);
  L.ssq = take(sizeof(float) * R * (d.H / 32 > 0 ? d.H / 32 : 1));
  {
    // split-K partials of the largest projection: (K / 256) slices x rows x columns
    const size_t a1 = (size_t)(d.H / 256) * (d.nqkv > 2 * d.F ? (d.nqkv > d.Vc ? d.nqkv : d.Vc) : (2 * d.F > d.Vc ? 2 * d.F : d.Vc));
    const size_t a2 = (size_t)(d.qd / 256) * d.H, a3 = (size_t)(d.F / 256) * d.H;
    const size_t mx = a1 > a2 ? (a1 > a3 ? a1 : a3) : (a2 > a3 ? a2 : a3);
    L.gpart = take(sizeof(float) * L.rows * (mx > 0 ? mx : 1));
  }
  {
    const int nmax = d.nqkv > d.F ? (d.nqkv > d.Vc ? d.nqkv : d.Vc) : (d.F > d.Vc ? d.F : d.Vc);
    // a counter per (32-column tile, 64-row block) of every projection
    L.gcnt_bytes = sizeof(uint32_t) * ((L.rows + 63) / 64) * (size_t)(nmax / 32 + 1 + (d.H / 32));
    L.gcnt = take(L.gcnt_bytes);
  }
  L.logits_t = take(sizeof(float) * (R > (size_t)B ? R : B) * d.Vc);
  L.logits_p = take(sizeof(float) * (size_t)(d.G - 1) * B * d.Vc);
  L.x0_dump = take(sizeof(float) * B * d.H);
  L.hidden_dump = take(sizeof(float) * (size_t)d.Lt * B * d.H);
  L.gather_dump = take(sizeof(int32_t) * B * (d.G + 1));
  L.tpos_dump = take(sizeof(int32_t) * B);
  // a call's padded chunk ids: at most PF_MAXROWS streams x (P + one chunk)
  const size_t pf_rows = (size_t)qtk::PF_MAXROWS * (d.P + kPrefillChunk);
  L.pf_codes = take(sizeof(int32_t) * pf_rows * d.G);
  L.pf_text = take(sizeof(int32_t) * pf_rows);
  L.pf_desc = take(sizeof(int32_t) * qtk::PF_WORDS);
  L.pf_xh = take(sizeof(float) * qtk::PF_MAXROWS * d.H);
  L.pf_lg = take(sizeof(float) * qtk::PF_MAXROWS * d.Vc);
  L.pf_br = take(sizeof(float) * qtk::PF_MAXROWS * d.H);
  L.ptab = take(sizeof(int32_t) * (size_t)B * d.P);
  L.f_tl = take(sizeof(qtk::LayerDev) * d.Lt);
  L.f_pl = take(sizeof(qtk::LayerDev) * d.Lp);
  L.f_heads = take(sizeof(void *) * d.G);
  L.f_heads_sc = take(sizeof(void *) * d.G);
  // rows every GEMV workgroup reads (residual, attention output, SiLU-mul
  // output) exist kXchRep times, one copy per group of readers
  L.xch_words = 2 * (size_t)d.H + 2 * (size_t)d.qd + 2 * (size_t)d.F + 32;
  L.f_xch_begin = off;  // every tagged exchange word lies in [f_xch_begin, f_err)
  L.f_xq = take(8 * kXchRep * L.xch_words);
  L.f_o = L.f_xq + 8 * 2 * (size_t)d.H;
  L.f_z = L.f_o + 8 * 2 * (size_t)d.qd;
  L.f_qkv = take(8 * 2 * (size_t)d.nqkv);
  L.f_amax = take(8 * 2 * (size_t)kMaxWG);
  L.f_lgx = take(8 * (size_t)d.Vc);
  L.f_part = take(8 * (size_t)d.nq * (d.P / kTile) * (d.hd + 2));
  L.f_err = take(64);
  L.f_trace = take(8 * 8 * 1024);
  L.total = off;
  return L;
}

size_t kv_elem(const qt_model_desc &m) { return m.kv_bf16 ? 2 : 4; }

size_t talker_ring_elems(const Dims &d, int32_t B) {
  return (size_t)B * d.Lt * 2 * d.kd * d.P;
}
// the paged talker ring: one pool of `rows` positions per (layer, K|V, head)
size_t talker_pool_elems(const Dims &d, int32_t rows) { return (size_t)d.Lt * 2 * d.kd * rows; }
size_t pred_ring_elems(const Dims &d, int32_t B) { return (size_t)B * d.Lp * 2 * d.kd * d.Q; }

// Shapes the kernels implement; message on failure.
const char *unsupported(const qt_model_desc &m) {
  const Dims d = dims_of(m);
  if (d.H <= 0 || d.nq <= 0 || d.nkv <= 0 || d.F <= 0 || d.Lt <= 0 || d.Lp <= 0 || d.Vc <= 0 ||
      d.Vt <= 0)
    return "non-positive model dimension";
  if (d.hd != 64 && d.hd != 128) return "head_dim must be 64 or 128";
  if (d.nq % d.nkv) return "n_kv_heads must divide n_q_heads";
  const int gq = d.nq / d.nkv;
  if (!(gq == 1 || gq == 2 || gq == 4) || gq * d.hd > 256) return "GQA group x head_dim must be <= 256 (group 1, 2 or 4)";
  if (d.G < 2 || d.G > 256) return "codebooks must be in [2, 256]";
  if (d.Q != d.G) return "predictor_positions must equal codebooks";
  if (d.P < kTile || d.P % kTile) return "talker_positions must be a positive multiple of 256";
  if (d.Q > d.P) return "predictor_positions exceeds talker_positions";
  if (m.lin_type < QT_LIN_F32 || m.lin_type > QT_LIN_Q4) return "unknown lin_type";
  const int ch = m.lin_type == QT_LIN_F32 ? 4 : (m.lin_type == QT_LIN_BF16 ? 8 : 32);
  if (d.H % ch || d.F % ch || d.qd % ch) return "hidden, ffn and n_q_heads*head_dim must be multiples of the weight chunk (4 f32, 8 bf16, 32 q8 / q4)";
  if (m.eps <= 0 || m.rope_theta <= 0) return "eps and rope_theta must be positive";
  return nullptr;
}

}  // namespace

struct qt_ctx {
  qt_model_desc md;
  Dims d;
  Layout L;
  int32_t B, K, maxF;
  uint32_t flags;
  hipStream_t stream;
  // weights (device pointers)
  const void *code_emb, *text_emb, *t_norm, *p_norm;
  qt_linear t_head;
  std::vector<qt_linear> p_heads;
  std::vector<qt_layer_weights> tl, pl;
  // device memory
  uint8_t *ring, *arena;
  // paged talker ring (QT_F_PAGED): pool rows, the host's free list and each
  // slot's rows by position (mirrored on the device in the page table)
  int32_t pool_rows = 0;
  std::vector<int32_t> free_rows;
  std::vector<std::vector<int32_t>> slot_rows;
  size_t pu_ptab = 0;
  // host mirrors and staging
  std::vector<int32_t> pos_host;
  std::vector<uint8_t> ready;
  // pinned staging (int32 elements): every async copy source has its own
  // region, so no host write can race a copy still in flight
  int32_t *pin_up = nullptr, *pin_down = nullptr;
  size_t pin_up_elems = 0, pin_down_elems = 0;
  size_t pu_ctl = 0, pu_overlay = 0, pu_forced = 0, pu_pf_text = 0, pu_pf_codes = 0, pu_scalar = 0;
  size_t pu_pf_desc = 0;  // one descriptor per prompt chunk of a call
  // prompt-chunk graphs by (streams, rows per stream, attention tiles, codes, head)
  std::map<uint64_t, std::pair<hipGraph_t, hipGraphExec_t>> pf_graphs;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  // adaptive K: a 1-frame graph for the frames of a call past its last
  // whole K-frame block (K > 1 only)
  hipGraph_t graph1 = nullptr;
  hipGraphExec_t exec1 = nullptr;
  int32_t path = QT_PATH_GRAPH;
  qtk::FrameArgs fa;       // persistent kernel arguments (path == QT_PATH_FRAME)
  int lds_limit = 0;       // LDS per workgroup on the device
  uint32_t tag_base = 1;   // running phase tag of the persistent kernel
  void *scratch = nullptr; // this device's static exchange region (qt_decode_frame_noalloc)
  float inv_temp = 0.f;    // sampling: float(1/T), 0 = greedy (sampler.h)
  int32_t top_k = 0;       // sampling: the k largest logits compete (0: all)
  uint64_t seed = 0;
  std::string err;

  template <class T> T *A(size_t off) const { return (T *)(arena + off); }
};

namespace {

// ----------------------------------------------------------------- paged ring
//
// With QT_F_PAGED the talker's K/V rows live in one pool shared by every slot,
// page size 1: each (slot, position) gets a pool row of its own from a host
// free list, and the device page table [B][P] (carried as data, like the
// set_rows destinations of [QT-log]) maps positions to rows, so a captured
// graph never changes.  Rows come from the free list as a slot's positions
// are first written and go back when the slot is prefilled again.

// Rows still to take for slot b to hold positions [0, upto).
size_t rows_short(const qt_ctx *c, int b, int upto) {
  const size_t have = c->slot_rows[b].size();
  return (size_t)upto > have ? (size_t)upto - have : 0;
}

// Give slot b rows for positions [0, upto) (the free list holds them: checked
// by the caller) and upload their table entries through `stage` (pinned).
hipError_t grow_slot(qt_ctx *c, int b, int upto, int32_t *stage) {
  std::vector<int32_t> &rows = c->slot_rows[b];
  const int first = (int)rows.size();
  if (upto <= first) return hipSuccess;
  for (int p = first; p < upto; ++p) {
    rows.push_back(c->free_rows.back());
    c->free_rows.pop_back();
    stage[p - first] = rows.back();
  }
  return hipMemcpyAsync(c->A<int32_t>(c->L.ptab) + (size_t)b * c->d.P + first, stage, sizeof(int32_t) * (upto - first),
                        hipMemcpyHostToDevice, c->stream);
}

// Return slot b's rows to the free list (host only).
void release_slot(qt_ctx *c, int b) {
  std::vector<int32_t> &rows = c->slot_rows[b];
  for (size_t i = rows.size(); i-- > 0;) c->free_rows.push_back(rows[i]);  // taken again in the same order
  rows.clear();
}

int32_t fail(qt_ctx *c, int32_t code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  g_err = buf;
  return code;
}

#define HIPCHK(ctx, expr)                                                              \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(ctx, QT_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));      \
  } while (0)

using namespace qtk;

int wtype_of(const qt_model_desc &m) {
  return m.lin_type == QT_LIN_F32 ? W_F32 : m.lin_type == QT_LIN_BF16 ? W_BF16 : m.lin_type == QT_LIN_Q8 ? W_Q8 : W_Q4;
}

Lin lin(const qt_linear &l) { return Lin{l.w, (const uint16_t *)l.scales}; }

// ----------------------------------------------------------------- schedule

struct Stack {
  const std::vector<qt_layer_weights> *layers;
  uint8_t *ring;          // (slot 0, layer 0, K) element base
  int64_t slot_stride;    // elements
  int64_t layer_stride;
  int64_t kv_stride;
  int32_t P;              // positions per head
  int32_t tile, max_tiles;
  const int32_t *ptab = nullptr;  // paged ring's page table (talker only)
  int32_t rows_per_head = 0;
};

Stack talker_stack(const qt_ctx *c) {
  const Dims &d = c->d;
  Stack s;
  s.layers = &c->tl;
  s.ring = c->ring;
  s.P = d.P;
  if (c->pool_rows) {  // paged: [Lt][2][nkv][pool rows][hd], rows from the page table
    s.kv_stride = (int64_t)d.kd * c->pool_rows;
    s.layer_stride = 2 * s.kv_stride;
    s.slot_stride = 0;
    s.ptab = c->A<int32_t>(c->L.ptab);
    s.rows_per_head = c->pool_rows;
  } else {
    s.kv_stride = (int64_t)d.kd * d.P;
    s.layer_stride = 2 * s.kv_stride;
    s.slot_stride = s.layer_stride * d.Lt;
    s.rows_per_head = d.P;
  }
  s.tile = kTile;
  s.max_tiles = c->L.max_tiles;
  return s;
}

Stack pred_stack(const qt_ctx *c) {
  const Dims &d = c->d;
  Stack s;
  s.layers = &c->pl;
  s.ring = c->ring + (c->pool_rows ? talker_pool_elems(d, c->pool_rows) : talker_ring_elems(d, c->B)) * kv_elem(c->md);
  s.rows_per_head = d.Q;
  s.kv_stride = (int64_t)d.kd * d.Q;
  s.layer_stride = 2 * s.kv_stride;
  s.slot_stride = s.layer_stride * d.Lp;
  s.P = d.Q;
  s.tile = d.Q;
  s.max_tiles = 1;
  return s;
}

// One decoder layer over M rows (x in the arena's activation rows).
// With bf16, q8 or q4 weights and bf16 operands, every projection of 1..512
// rows goes through the split-K MFMA GEMM: even at one row it spreads each
// weight row's K over its workgroups, where the GEMV gives a row to one wave
// (a 1,024-wide q4 row fills only half of it).  F32 models use the GEMV.
// The choice is made once per model, never per projection: the GEMM's
// RMSNorm reads the row sums of squares that the GEMM's residual epilogues
// (and the gather / argmax kernels) leave, which the GEMV's residual epilogue
// does not write, so a model whose hidden, attention or FFN width is not a
// multiple of the GEMM's 256-wide K slice runs every projection on the GEMV.
bool model_uses_gemm(const qt_model_desc &md, const Dims &d) {
  return md.lin_type != QT_LIN_F32 && md.act_bf16 && d.H % 256 == 0 && d.qd % 256 == 0 && d.F % 256 == 0 &&
         d.nqkv % 32 == 0 && d.Vc % 32 == 0;
}
bool use_gemm(const qt_ctx *c, int M) {
  return model_uses_gemm(c->md, c->d) && M >= 1 && M <= std::min(c->L.rows, qtk::GEMM_MAX_ROWS);
}

// One projection.  ssq_in: the input rows' sums of squares in 32-column slots
// (row m at ssq_in + m * ssq_stride), needed by the GEMM's RMSNorm; ssq_out:
// where a residual epilogue leaves the new rows' sums.
// kpw: 256-wide K slices per GEMM workgroup (fewer split-K partials; taken
// only where it divides the projection's K slices).
hipError_t project(qt_ctx *c, int epi, const GemvArgs &g, const float *ssq_in, int ssq_stride, float *ssq_out,
                   int kpw = 1) {
  const int wt = wtype_of(c->md);
  if (!use_gemm(c, g.M)) return launch_gemv(wt, epi, g, c->stream);
  GemmArgs a = {};
  for (int i = 0; i < 3; ++i) { a.seg[i] = g.seg[i]; a.seg_end[i] = g.seg_end[i]; }
  a.nseg = g.nseg; a.up = g.up;
  a.N = g.N; a.K = g.K; a.M = g.M;
  a.x = g.x; a.x_stride = g.x_stride;
  a.gain = g.gain; a.gain_bf16 = g.gain_bf16; a.eps = g.eps;
  a.ssq = ssq_in; a.ssq_stride = ssq_stride;
  a.y = g.y; a.y_stride = g.y_stride;
  a.ssq_out = ssq_out; a.normed_out = g.normed_out;
  a.copy_out = g.copy_out; a.copy_stride = g.copy_stride;
  a.part = c->A<float>(c->L.gpart);
  a.cnt = c->A<uint32_t>(c->L.gcnt);
  a.kpw = (g.K / 256) % kpw == 0 ? kpw : 1;
  return launch_gemm(wt, epi, a, c->stream);
}

hipError_t enqueue_layer(qt_ctx *c, const Stack &st, int l, int M, const RowMap &rows,
                         float *hidden_copy) {
  const Dims &d = c->d;
  const qt_model_desc &md = c->md;
  const qt_layer_weights &w = (*st.layers)[l];
  const int wt = wtype_of(md);
  hipStream_t s = c->stream;
  float *x = c->A<float>(c->L.x);
  float *qkv = c->A<float>(c->L.qkv);
  float *q = c->A<float>(c->L.q);
  float *o = c->A<float>(c->L.o);
  float *z = c->A<float>(c->L.z);
  uint8_t *ring_layer = st.ring + (size_t)l * st.layer_stride * kv_elem(md);
  hipError_t e;

  GemvArgs g = {};
  g.act_bf16 = md.act_bf16;
  g.gain_bf16 = md.tab_bf16;
  g.eps = (float)md.eps;
  // prompt chunks (16 to 512 rows) take two K slices per GEMM workgroup,
  // every chunk alike, so a row's bits do not depend on how its prompt is cut
  const int kpw = rows.pf ? kPfSlicesPerWg : 1;

  // 1. QKV with the attention RMSNorm prologue
  g.seg[0] = lin(w.wq); g.seg[1] = lin(w.wk); g.seg[2] = lin(w.wv);
  g.seg_end[0] = d.qd; g.seg_end[1] = d.qd + d.kd; g.seg_end[2] = d.nqkv;
  g.nseg = 3;
  g.N = d.nqkv; g.K = d.H;
  g.x = x; g.x_stride = d.H; g.M = M;
  g.gain = w.attn_norm;
  g.y = qkv; g.y_stride = d.nqkv;
  float *ssq = c->A<float>(c->L.ssq);
  const int ss = d.H / 32;
  if ((e = project(c, EPI_STORE, g, ssq, ss, nullptr, kpw)) != hipSuccess) return e;

  // 2. q/k norm + RoPE + K/V rows into the ring at the row's position: the
  // attention tile's prologue for the predictor's decode steps (one tile per
  // row, latency-bound); a kernel of its own for prefill chunks, for the
  // talker, whose long tiles stream K/V at a higher occupancy without it, and
  // for a paged ring (the fused prologue writes the dense cache only)
  const bool fused = rows.rows_per_slot <= 2 && st.max_tiles == 1 && !st.ptab;
  if (!fused) {
    QkArgs qa = {};
    qa.qkv = qkv; qa.M = M; qa.rows = rows; qa.nq = d.nq; qa.nkv = d.nkv;
    qa.q_gain = w.q_norm; qa.k_gain = w.k_norm; qa.gain_bf16 = md.tab_bf16; qa.eps = (float)md.eps;
    qa.rope_cos = c->A<float>(c->L.rope_cos); qa.rope_sin = c->A<float>(c->L.rope_sin);
    qa.q_out = q; qa.ring_layer = ring_layer; qa.slot_stride = st.slot_stride;
    qa.kv_stride = st.kv_stride; qa.P = st.P; qa.ptab = st.ptab; qa.rows_per_head = st.rows_per_head;
    if ((e = launch_qk_rope_kv(d.hd, md.kv_bf16, qa, s)) != hipSuccess) return e;
  }

  // 3. attention over the (padded) window
  AttnArgs aa = {};
  if (fused) {
    aa.qkv = qkv;
    aa.q_gain = w.q_norm; aa.k_gain = w.k_norm; aa.gain_bf16 = md.tab_bf16; aa.eps = (float)md.eps;
    aa.rope_cos = c->A<float>(c->L.rope_cos); aa.rope_sin = c->A<float>(c->L.rope_sin);
  }
  aa.q = q; aa.M = M; aa.rows = rows; aa.nq = d.nq; aa.nkv = d.nkv;
  aa.ring_layer = ring_layer; aa.slot_stride = st.slot_stride; aa.kv_stride = st.kv_stride;
  aa.P = st.P; aa.tile = st.tile; aa.max_tiles = st.max_tiles;
  aa.ptab = st.ptab; aa.rows_per_head = st.rows_per_head;
  // rows with host-known positions (prefill chunks, the predictor) launch only
  // the tiles up to their last position, and skip the merge when that is one
  aa.grid_tiles = rows.pos_dev ? st.max_tiles
                               : std::min(st.max_tiles, (rows.pos_base + rows.rows_per_slot - 1) / st.tile + 1);
  aa.scale = (float)(1.0 / sqrt((double)d.hd));
  aa.o = o; aa.part = c->A<float>(c->L.part);
  // prompt chunks: 16 query positions per workgroup on MFMA where the shape
  // allows (hd 128, bf16 cache; the group is then 1 or 2), else the decode tiles
  const int gq = d.nq / d.nkv;
  if (rows.pf && d.hd == 128 && md.kv_bf16 && (gq == 1 || gq == 2)) {
    if ((e = launch_attn_prompt(d.hd, md.kv_bf16, aa, M / rows.rows_per_slot, s)) != hipSuccess) return e;
  } else if ((e = launch_attention(d.hd, md.kv_bf16, aa, aa.grid_tiles > 1, s)) != hipSuccess) {
    return e;
  }

  // 4. O projection, residual added in the epilogue
  GemvArgs go = g;
  go.seg[0] = lin(w.wo); go.nseg = 1; go.seg_end[0] = d.H;
  go.N = d.H; go.K = d.qd; go.x = o; go.x_stride = d.qd; go.gain = nullptr;
  go.y = x; go.y_stride = d.H;
  if ((e = project(c, EPI_RESID, go, nullptr, 0, ssq, kpw)) != hipSuccess) return e;

  // 5. gate/up with the MLP RMSNorm prologue, SiLU-multiply epilogue
  GemvArgs gu = g;
  gu.seg[0] = lin(w.wg); gu.up = lin(w.wu); gu.nseg = 1; gu.seg_end[0] = d.F;
  gu.N = d.F; gu.K = d.H; gu.x = x; gu.x_stride = d.H; gu.gain = w.mlp_norm;
  gu.y = z; gu.y_stride = d.F;
  if ((e = project(c, EPI_GATED, gu, ssq, ss, nullptr, kpw)) != hipSuccess) return e;

  // 6. down projection, residual added in the epilogue
  GemvArgs gd = g;
  gd.seg[0] = lin(w.wd); gd.nseg = 1; gd.seg_end[0] = d.H;
  gd.N = d.H; gd.K = d.F; gd.x = z; gd.x_stride = d.F; gd.gain = nullptr;
  gd.y = x; gd.y_stride = d.H;
  gd.copy_out = hidden_copy; gd.copy_stride = d.H;
  return project(c, EPI_RESID, gd, nullptr, 0, ssq, kpw);
}

// Frame k of a replay: predictor (codes 1..G-1) then the talker step.
hipError_t enqueue_frame(qt_ctx *c, int k) {
  const Dims &d = c->d;
  const qt_model_desc &md = c->md;
  const int B = c->B;
  const int wt = wtype_of(md);
  const bool dump = c->flags & QT_F_DUMP;
  hipStream_t s = c->stream;
  float *x = c->A<float>(c->L.x);
  int32_t *ctl = c->A<int32_t>(c->L.ctl);
  hipError_t e;

  // predictor prefill rows [bridge, E_0[c0]] ([QT-log] set_rows / bridge entry)
  PredInArgs pa = {};
  pa.bridge = c->A<float>(c->L.bridge); pa.code_emb = c->code_emb; pa.tab_bf16 = md.tab_bf16;
  pa.H = d.H; pa.G = d.G; pa.B = B; pa.c0_state = c->A<int32_t>(c->L.c0); pa.ctl = ctl; pa.k = k;
  pa.cin = c->A<int32_t>(c->L.cin); pa.cout = c->A<int32_t>(c->L.cout); pa.x = x;
  float *ssq = c->A<float>(c->L.ssq);
  const int ss = d.H / 32;
  pa.ssq = ssq;
  if ((e = launch_pred_input(pa, s)) != hipSuccess) return e;

  const Stack ps = pred_stack(c);
  for (int j = 0; j < d.G - 1; ++j) {
    // j == 0: two rows per stream at positions 0, 1; else one row at j + 1
    // ([QT-log] per-layer K/V ring entry: T=2 prefill then single-row decodes)
    const int M = j == 0 ? 2 * B : B;
    const RowMap rows = j == 0 ? RowMap{0, 2, 0, nullptr} : RowMap{0, 1, j + 1, nullptr};
    for (int l = 0; l < d.Lp; ++l)
      if ((e = enqueue_layer(c, ps, l, M, rows, nullptr)) != hipSuccess) return e;
    GemvArgs h = {};
    h.seg[0] = lin(c->p_heads[j]); h.nseg = 1; h.seg_end[0] = d.Vc;
    h.N = d.Vc; h.K = d.H;
    h.x = j == 0 ? x + d.H : x; h.x_stride = j == 0 ? 2 * d.H : d.H; h.M = B;
    h.gain = c->p_norm; h.gain_bf16 = md.tab_bf16; h.eps = (float)md.eps; h.act_bf16 = md.act_bf16;
    float *lg = c->A<float>(c->L.logits_p) + (size_t)j * B * d.Vc;
    h.y = lg; h.y_stride = d.Vc;
    if ((e = project(c, EPI_STORE, h, j == 0 ? ssq + ss : ssq, j == 0 ? 2 * ss : ss, nullptr)) != hipSuccess) return e;
    ArgmaxArgs am = {};
    am.logits = lg; am.Vc = d.Vc; am.M = B; am.mode = AM_PRED; am.j = j; am.ctl = ctl; am.k = k;
    am.pos = c->A<int32_t>(c->L.pos);
    am.B = B; am.G = d.G; am.cin = pa.cin; am.cout = pa.cout; am.code_emb = c->code_emb;
    am.tab_bf16 = md.tab_bf16; am.H = d.H; am.x_next = x; am.ssq = ssq;
    if ((e = launch_argmax(am, s)) != hipSuccess) return e;
  }

  // talker step: gather-sum of the frame's codes + overlay ([QT-log] AR inputs entry)
  GatherArgs ga = {};
  ga.code_emb = c->code_emb; ga.text_emb = c->text_emb; ga.tab_bf16 = md.tab_bf16;
  ga.H = d.H; ga.Vc = d.Vc; ga.G = d.G;
  ga.codes = c->A<int32_t>(c->L.cin) + (size_t)k * B * d.G; ga.codes_stride = d.G;
  ga.text = c->A<int32_t>(c->L.overlay) + (size_t)k * B; ga.text_stride = 1;
  ga.ctl = ctl; ga.frame_stride_codes = B * d.G; ga.frame_stride_text = B;
  ga.x = x; ga.M = B;
  ga.x0_dump = dump ? c->A<float>(c->L.x0_dump) : nullptr;
  ga.gather_dump = dump ? c->A<int32_t>(c->L.gather_dump) : nullptr;
  ga.ssq = ssq;
  if ((e = launch_gather(ga, s)) != hipSuccess) return e;

  const Stack ts = talker_stack(c);
  const RowMap trows{0, 1, 0, c->A<int32_t>(c->L.pos)};
  for (int l = 0; l < d.Lt; ++l) {
    float *hc = dump ? c->A<float>(c->L.hidden_dump) + (size_t)l * B * d.H : nullptr;
    if ((e = enqueue_layer(c, ts, l, B, trows, hc)) != hipSuccess) return e;
  }
  // final norm -> bridge (kept on device), head, argmax -> next c0, pos += 1
  GemvArgs h = {};
  h.seg[0] = lin(c->t_head); h.nseg = 1; h.seg_end[0] = d.Vc;
  h.N = d.Vc; h.K = d.H; h.x = x; h.x_stride = d.H; h.M = B;
  h.gain = c->t_norm; h.gain_bf16 = md.tab_bf16; h.eps = (float)md.eps; h.act_bf16 = md.act_bf16;
  h.normed_out = c->A<float>(c->L.bridge);
  h.y = c->A<float>(c->L.logits_t); h.y_stride = d.Vc;
  if ((e = project(c, EPI_STORE, h, ssq, ss, nullptr)) != hipSuccess) return e;
  ArgmaxArgs am = {};
  am.logits = h.y; am.Vc = d.Vc; am.M = B; am.mode = AM_TALKER; am.ctl = ctl; am.k = k;
  am.B = B; am.G = d.G; am.c0_state = c->A<int32_t>(c->L.c0); am.pos = c->A<int32_t>(c->L.pos);
  am.tpos_dump = dump ? c->A<int32_t>(c->L.tpos_dump) : nullptr;
  return launch_argmax(am, s);
}

// ----------------------------------------------------------------- prompt chunks
//
// A prompt is prefilled in chunks of up to kPrefillChunk rows ([QT-log]
// per-layer K/V ring entry: the prefill writes positions [0, T)).  One call
// takes 1-4 streams ([MC-opt] round-18 table, talker chunk-prefill graphs: a
// graph per row count and token bucket): each chunk holds the same t
// positions [r0, r0 + t) of every stream whose prompt is still going, t a
// token bucket (a power of two from 16, at most kPrefillChunk rows in all),
// a shorter prompt's rows past its end being padding that reaches neither
// the ring nor the result.  Every weight matrix is read once per chunk, so
// long prompts take the largest chunks the batched GEMM holds.  The
// chunk's ids, slots and positions live in a device descriptor, so one
// captured graph per (streams, t, attention tiles, codes given, head)
// serves every chunk of that shape; the chunk in which a stream's prompt
// ends also runs the head and decides the stream's first code (c0).

struct PfShape {
  int n, t, r0, tiles;  // r0: the chunk start the capture sizes the attention grid from
  bool codes, head;
  uint64_t key() const {  // fields wide enough for any n, t and tile count
    return (uint64_t)n | (uint64_t)t << 8 | (uint64_t)tiles << 24 | (uint64_t)codes << 48 | (uint64_t)head << 49;
  }
};

hipError_t enqueue_pf_chunk(qt_ctx *c, const PfShape &sh) {
  const Dims &d = c->d;
  const qt_model_desc &md = c->md;
  hipStream_t s = c->stream;
  const int32_t *pf = c->A<int32_t>(c->L.pf_desc);
  float *x = c->A<float>(c->L.x);
  const int M = sh.n * sh.t;
  hipError_t e;
  // gather-sum of the chunk's rows ([QT-log] AR inputs entry); the ids start
  // at the descriptor's PF_IDOFF row
  GatherArgs ga = {};
  ga.code_emb = c->code_emb; ga.text_emb = c->text_emb; ga.tab_bf16 = md.tab_bf16;
  ga.H = d.H; ga.Vc = d.Vc; ga.G = d.G;
  ga.codes = sh.codes ? c->A<int32_t>(c->L.pf_codes) : nullptr; ga.codes_stride = d.G;
  ga.text = c->A<int32_t>(c->L.pf_text); ga.text_stride = 1;
  ga.ctl = pf; ga.frame_stride_codes = d.G; ga.frame_stride_text = 1;
  ga.x = x; ga.M = M; ga.ssq = c->A<float>(c->L.ssq);
  if ((e = launch_gather(ga, s)) != hipSuccess) return e;
  const Stack ts = talker_stack(c);
  RowMap rows{0, sh.t, sh.r0, nullptr};
  rows.pf = pf;
  for (int l = 0; l < d.Lt; ++l)
    if ((e = enqueue_layer(c, ts, l, M, rows, nullptr)) != hipSuccess) return e;
  if (!sh.head) return hipSuccess;
  // final norm -> bridge, head, first code of the streams whose prompt ends here
  float *xh = c->A<float>(c->L.pf_xh);
  if ((e = launch_pf_rows(pf, x, xh, sh.n, d.H, s)) != hipSuccess) return e;
  GemvArgs h = {};
  h.seg[0] = lin(c->t_head); h.nseg = 1; h.seg_end[0] = d.Vc;
  h.N = d.Vc; h.K = d.H; h.x = xh; h.x_stride = d.H; h.M = sh.n;
  h.gain = c->t_norm; h.gain_bf16 = md.tab_bf16; h.eps = (float)md.eps; h.act_bf16 = md.act_bf16;
  h.normed_out = c->A<float>(c->L.pf_br);
  h.y = c->A<float>(c->L.pf_lg); h.y_stride = d.Vc;
  if ((e = launch_gemv(wtype_of(md), EPI_STORE, h, s)) != hipSuccess) return e;
  ArgmaxArgs am = {};
  am.logits = h.y; am.Vc = d.Vc; am.M = sh.n; am.mode = AM_PREFILL; am.ctl = pf;
  am.c0_state = c->A<int32_t>(c->L.c0); am.pos = c->A<int32_t>(c->L.pos);
  am.bridge_src = h.normed_out; am.bridge = c->A<float>(c->L.bridge); am.H = d.H;
  am.logits_out = c->A<float>(c->L.logits_t);
  return launch_argmax(am, s);
}

// kf frames (a replay of the K-frame graph, or the 1-frame one)
hipError_t enqueue_replay(qt_ctx *c, int kf) {
  hipError_t e;
  for (int k = 0; k < kf; ++k)
    if ((e = enqueue_frame(c, k)) != hipSuccess) return e;
  return launch_advance(c->A<int32_t>(c->L.ctl), kf, c->stream);
}

const char *frame_unsupported(const qt_model_desc &m, int B) {
  const Dims d = dims_of(m);
  if (B != 1) return "the persistent kernel decodes one stream";
  if (!qtk::frame_variant_supported(wtype_of(m), d.hd, d.nq / d.nkv, m.kv_bf16)) return "no persistent-kernel variant";
  if (m.lin_type != QT_LIN_F32 && !(m.act_bf16 && m.tab_bf16)) return "bf16/q8/q4 weights need bf16 operands and tables";
  if (m.lin_type == QT_LIN_F32 && (m.act_bf16 || m.tab_bf16)) return "f32 weights need f32 operands and tables";
  return nullptr;
}

int32_t prefill_rows(qt_ctx *c, int32_t n, const int32_t *slots, const int32_t *lens, const int32_t *codes,
                     const int32_t *text_ids);
int32_t decode_chunks(qt_ctx *c, int32_t n, const int32_t *overlay_ids, int32_t *codes_out,
                      const int32_t *forced, bool static_scratch);
int32_t decode_entry(qt_ctx *c, int32_t n, const int32_t *overlay_ids, int32_t *codes_out, const int32_t *forced,
                     bool static_scratch);

bool ids_ok(const int32_t *p, size_t n, int32_t hi) {
  for (size_t i = 0; i < n; ++i)
    if (p[i] < 0 || p[i] >= hi) return false;
  return true;
}

}  // namespace

// ----------------------------------------------------------------- C ABI

extern "C" {

int32_t qt_abi_version(void) { return QT_ABI_VERSION; }

int32_t qt_path(const qt_ctx *ctx) { return ctx ? ctx->path : QT_E_ARG; }

int32_t qt_set_sampler(qt_ctx *c, float temperature, int32_t top_k, uint64_t seed) {
  if (!c) return fail(nullptr, QT_E_ARG, "NULL context");
  if (!(temperature >= 0.f) || isinf(temperature))
    return fail(c, QT_E_ARG, "temperature must be finite and >= 0");
  if (top_k < 0) return fail(c, QT_E_ARG, "top_k must be >= 0");
  if (top_k > 0 && top_k < c->d.Vc && c->d.Vc > 2048)
    return fail(c, QT_E_UNSUPPORTED, "top-k supports codebooks of at most 2048 entries");
  c->inv_temp = temperature > 0.f ? (float)(1.0 / (double)temperature) : 0.f;
  c->top_k = top_k;
  c->seed = seed;
  return QT_OK;
}

const char *qt_last_error(const qt_ctx *ctx) { return ctx ? ctx->err.c_str() : g_err.c_str(); }

int32_t qt_query_sizes(const qt_model_desc *model, int32_t max_batch, int32_t frames_per_replay,
                       int32_t max_frames_per_call, uint32_t flags, size_t *ring_bytes,
                       size_t *arena_bytes) {
  if (!model || !ring_bytes || !arena_bytes) return fail(nullptr, QT_E_ARG, "NULL argument");
  if (max_batch <= 0 || frames_per_replay <= 0 || max_frames_per_call <= 0)
    return fail(nullptr, QT_E_ARG, "max_batch, frames_per_replay and max_frames_per_call must be positive");
  if (max_frames_per_call % frames_per_replay)
    return fail(nullptr, QT_E_ARG, "max_frames_per_call must be a multiple of frames_per_replay");
  if (flags & ~(QT_F_DUMP | QT_F_EAGER | QT_F_OPS | QT_F_TRACE | QT_F_PAGED)) return fail(nullptr, QT_E_ARG, "unknown flags");
  if (const char *why = unsupported(*model)) return fail(nullptr, QT_E_UNSUPPORTED, "%s", why);
  const Dims d = dims_of(*model);
  *ring_bytes = (talker_ring_elems(d, max_batch) + pred_ring_elems(d, max_batch)) * kv_elem(*model);
  *arena_bytes = layout_of(d, max_batch, max_frames_per_call).total;
  return QT_OK;
}

int32_t qt_query_paged_ring(const qt_model_desc *model, int32_t max_batch, int32_t pool_rows, size_t *ring_bytes) {
  if (!model || !ring_bytes) return fail(nullptr, QT_E_ARG, "NULL argument");
  if (max_batch <= 0 || pool_rows <= 0) return fail(nullptr, QT_E_ARG, "max_batch and pool_rows must be positive");
  if (const char *why = unsupported(*model)) return fail(nullptr, QT_E_UNSUPPORTED, "%s", why);
  const Dims d = dims_of(*model);
  *ring_bytes = (talker_pool_elems(d, pool_rows) + pred_ring_elems(d, max_batch)) * kv_elem(*model);
  return QT_OK;
}

void qt_free(qt_ctx *c) {
  if (!c) return;
  if (c->exec) (void)hipGraphExecDestroy(c->exec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  if (c->exec1) (void)hipGraphExecDestroy(c->exec1);
  if (c->graph1) (void)hipGraphDestroy(c->graph1);
  for (auto &kv : c->pf_graphs) {
    (void)hipGraphExecDestroy(kv.second.second);
    (void)hipGraphDestroy(kv.second.first);
  }
  if (c->pin_up) (void)hipHostFree(c->pin_up);
  if (c->pin_down) (void)hipHostFree(c->pin_down);
  delete c;
}

int32_t qt_init(const qt_init_params *params, qt_ctx **out) {
  if (!params || !out) return fail(nullptr, QT_E_ARG, "NULL argument");
  if (params->abi_version < QT_ABI_MIN_VERSION || params->abi_version > QT_ABI_VERSION)
    return fail(nullptr, QT_E_ABI, "abi_version %u outside [%d, %d]", params->abi_version,
                QT_ABI_MIN_VERSION, QT_ABI_VERSION);
  // callers of ABI 1-3 pass the structure without pool_rows (a dense ring)
  const size_t old_size = offsetof(qt_init_params, pool_rows);
  if (params->struct_size != sizeof(qt_init_params) && params->struct_size != old_size)
    return fail(nullptr, QT_E_ARG, "struct_size %u is neither %zu nor %zu", params->struct_size,
                sizeof(qt_init_params), old_size);
  qt_init_params pv = {};
  memcpy(&pv, params, params->struct_size);
  const qt_init_params *p = &pv;
  const bool paged = (p->flags & QT_F_PAGED) != 0;
  if (paged && p->pool_rows <= 0) return fail(nullptr, QT_E_ARG, "QT_F_PAGED needs pool_rows > 0");
  size_t ring_need, arena_need;
  int32_t rc = qt_query_sizes(&p->model, p->max_batch, p->frames_per_replay,
                              p->max_frames_per_call, p->flags, &ring_need, &arena_need);
  if (rc != QT_OK) return rc;
  if (paged && (rc = qt_query_paged_ring(&p->model, p->max_batch, p->pool_rows, &ring_need)) != QT_OK) return rc;
  const qt_model_desc &m = p->model;
  const Dims d = dims_of(m);
  const qt_weights &w = p->weights;
  if (!p->ring || !p->arena) return fail(nullptr, QT_E_ARG, "NULL ring or arena");
  if (((uintptr_t)p->ring | (uintptr_t)p->arena) % kAlign)
    return fail(nullptr, QT_E_ARG, "ring and arena must be 256-byte aligned");
  if (p->ring_bytes < ring_need || p->arena_bytes < arena_need)
    return fail(nullptr, QT_E_SIZE, "ring %zu < %zu or arena %zu < %zu bytes", p->ring_bytes,
                ring_need, p->arena_bytes, arena_need);
  if (!p->stream && !(p->flags & QT_F_EAGER))
    return fail(nullptr, QT_E_ARG, "graph replay needs a non-default stream (or QT_F_EAGER)");
  if (!w.code_emb || !w.text_emb || !w.talker || !w.talker_norm || !w.talker_head.w ||
      !w.predictor || !w.predictor_norm || !w.predictor_heads)
    return fail(nullptr, QT_E_ARG, "NULL weight pointer");
  const bool blocked = m.lin_type == QT_LIN_Q8 || m.lin_type == QT_LIN_Q4;
  auto lin_ok = [&](const qt_linear &l) {
    if (!l.w || (blocked && !l.scales)) return false;
    if ((uintptr_t)l.w % 16) return false;  // 128-bit loads
    return true;
  };
  auto layer_ok = [&](const qt_layer_weights &L) {
    return L.attn_norm && L.q_norm && L.k_norm && L.mlp_norm && lin_ok(L.wq) && lin_ok(L.wk) &&
           lin_ok(L.wv) && lin_ok(L.wo) && lin_ok(L.wg) && lin_ok(L.wu) && lin_ok(L.wd);
  };
  for (int l = 0; l < d.Lt; ++l)
    if (!layer_ok(w.talker[l])) return fail(nullptr, QT_E_ARG, "talker layer %d: NULL or unaligned weight", l);
  for (int l = 0; l < d.Lp; ++l)
    if (!layer_ok(w.predictor[l])) return fail(nullptr, QT_E_ARG, "predictor layer %d: NULL or unaligned weight", l);
  if (!lin_ok(w.talker_head)) return fail(nullptr, QT_E_ARG, "talker head: NULL or unaligned");
  for (int j = 0; j < d.G - 1; ++j)
    if (!lin_ok(w.predictor_heads[j])) return fail(nullptr, QT_E_ARG, "predictor head %d: NULL or unaligned", j);

  qt_ctx *c = new qt_ctx();
  c->md = m;
  c->d = d;
  c->B = p->max_batch;
  c->K = p->frames_per_replay;
  c->maxF = p->max_frames_per_call;
  c->flags = p->flags;
  c->stream = (hipStream_t)p->stream;
  c->L = layout_of(d, c->B, c->maxF);
  c->code_emb = w.code_emb; c->text_emb = w.text_emb;
  c->t_norm = w.talker_norm; c->p_norm = w.predictor_norm; c->t_head = w.talker_head;
  c->tl.assign(w.talker, w.talker + d.Lt);
  c->pl.assign(w.predictor, w.predictor + d.Lp);
  c->p_heads.assign(w.predictor_heads, w.predictor_heads + d.G - 1);
  c->ring = (uint8_t *)p->ring;
  c->arena = (uint8_t *)p->arena;
  c->pos_host.assign(c->B, 0);
  c->ready.assign(c->B, 0);
  if (paged) {
    c->pool_rows = p->pool_rows;
    c->free_rows.resize(p->pool_rows);
    for (int32_t i = 0; i < p->pool_rows; ++i) c->free_rows[i] = p->pool_rows - 1 - i;  // row 0 is taken first
    c->slot_rows.assign(c->B, {});
  }

  auto bail = [&](int32_t code) {
    g_err = c->err;
    qt_free(c);
    return code;
  };
  // pinned staging: ctl + overlay + forced codes + prefill ids up; codes down
  c->pu_ctl = 0;
  c->pu_overlay = 16;
  c->pu_forced = c->pu_overlay + (size_t)c->maxF * c->B;
  const size_t pf_rows = (size_t)qtk::PF_MAXROWS * (d.P + kPrefillChunk);
  c->pu_pf_text = c->pu_forced + (size_t)c->maxF * c->B * d.G;
  c->pu_pf_codes = c->pu_pf_text + pf_rows;
  c->pu_pf_desc = c->pu_pf_codes + pf_rows * d.G;
  c->pu_scalar = c->pu_pf_desc + (size_t)(d.P / kPfMinRows + 2) * qtk::PF_WORDS;
  // paged: new table entries (a prefill's streams' P each, or maxF per slot per decode chunk)
  c->pu_ptab = c->pu_scalar + 16;
  c->pin_up_elems = c->pu_ptab + std::max((size_t)qtk::PF_MAXROWS * d.P, (size_t)c->maxF * c->B);
  c->pin_down_elems = (size_t)c->maxF * c->B * d.G;
  if (hipHostMalloc((void **)&c->pin_up, c->pin_up_elems * 4, hipHostMallocDefault) != hipSuccess ||
      hipHostMalloc((void **)&c->pin_down, c->pin_down_elems * 4, hipHostMallocDefault) != hipSuccess)
    return bail(fail(c, QT_E_HIP, "hipHostMalloc of staging buffers failed"));

  // RoPE table: angle p * theta^(-2i/hd) in double, cos/sin rounded to f32
  {
    const int h = d.hd / 2;
    std::vector<float> cs((size_t)d.P * h), sn((size_t)d.P * h);
    for (int pp = 0; pp < d.P; ++pp)
      for (int i = 0; i < h; ++i) {
        const double ang = (double)pp * pow(m.rope_theta, -2.0 * i / (double)d.hd);
        cs[(size_t)pp * h + i] = (float)cos(ang);
        sn[(size_t)pp * h + i] = (float)sin(ang);
      }
    if (hipMemcpyAsync(c->arena + c->L.rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, c->stream) != hipSuccess ||
        hipMemcpyAsync(c->arena + c->L.rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, c->stream) != hipSuccess ||
        hipStreamSynchronize(c->stream) != hipSuccess)
      return bail(fail(c, QT_E_HIP, "RoPE table upload failed"));
  }
  // the batched projections' tile counters start at zero (their last workgroup resets them);
  // cleared here, before any capture
  if (hipMemsetAsync(c->arena + c->L.gcnt, 0, c->L.gcnt_bytes, c->stream) != hipSuccess ||
      hipStreamSynchronize(c->stream) != hipSuccess)
    return bail(fail(c, QT_E_HIP, "counter clear failed"));
  // decode path: persistent frame kernel where it applies
  c->path = (c->flags & QT_F_EAGER) ? QT_PATH_EAGER : QT_PATH_GRAPH;
  if (!(c->flags & (QT_F_EAGER | QT_F_OPS | QT_F_PAGED)) && !frame_unsupported(m, c->B)) {
    int dev = 0, ncu = 0;
    const char *why = nullptr;
    int lds = 0;
    qtk::FrameArgs &fa = c->fa;
    fa = qtk::FrameArgs{};
    fa.H = d.H; fa.nq = d.nq; fa.nkv = d.nkv; fa.hd = d.hd; fa.F = d.F; fa.Lt = d.Lt; fa.Lp = d.Lp;
    fa.G = d.G; fa.Vc = d.Vc; fa.Vt = d.Vt; fa.P = d.P; fa.Q = d.Q;
    fa.wt = wtype_of(m); fa.tab_bf16 = m.tab_bf16; fa.kv_bf16 = m.kv_bf16; fa.act_bf16 = m.act_bf16;
    fa.rep = kXchRep; fa.rep_stride = (int64_t)c->L.xch_words;
    // the plan must fit for the longest context the ring holds
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
        ncu > 0 && ncu <= kMaxWG && (fa.nwg = ncu, qtk::frame_plan(fa, d.P - 1, lds, &why)) &&
        qtk::frame_coresident(fa, ncu)) {
      c->lds_limit = lds;
      fa.eps = (float)m.eps; fa.scale = (float)(1.0 / sqrt((double)d.hd));
      // device-side weight tables
      std::vector<qtk::LayerDev> tl(d.Lt), pl(d.Lp);
      auto fill = [&](qtk::LayerDev &o, const qt_layer_weights &L) {
        o.attn_norm = L.attn_norm; o.q_norm = L.q_norm; o.k_norm = L.k_norm; o.mlp_norm = L.mlp_norm;
        const qt_linear *ls[7] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.wg, &L.wu, &L.wd};
        for (int i = 0; i < 7; ++i) { o.w[i] = ls[i]->w; o.sc[i] = (const uint16_t *)ls[i]->scales; }
      };
      for (int l = 0; l < d.Lt; ++l) fill(tl[l], c->tl[l]);
      for (int l = 0; l < d.Lp; ++l) fill(pl[l], c->pl[l]);
      std::vector<const void *> hw(d.G), hs(d.G);
      hw[0] = c->t_head.w; hs[0] = c->t_head.scales;
      for (int j = 0; j < d.G - 1; ++j) { hw[j + 1] = c->p_heads[j].w; hs[j + 1] = c->p_heads[j].scales; }
      if (hipMemcpy(c->arena + c->L.f_tl, tl.data(), sizeof(qtk::LayerDev) * d.Lt, hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy(c->arena + c->L.f_pl, pl.data(), sizeof(qtk::LayerDev) * d.Lp, hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy(c->arena + c->L.f_heads, hw.data(), sizeof(void *) * d.G, hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy(c->arena + c->L.f_heads_sc, hs.data(), sizeof(void *) * d.G, hipMemcpyHostToDevice) != hipSuccess)
        return bail(fail(c, QT_E_HIP, "frame table upload failed"));
      fa.tl = c->A<qtk::LayerDev>(c->L.f_tl);
      fa.pl = c->A<qtk::LayerDev>(c->L.f_pl);
      fa.code_emb = c->code_emb; fa.text_emb = c->text_emb; fa.t_norm = c->t_norm; fa.p_norm = c->p_norm;
      fa.head_w = c->A<const void *>(c->L.f_heads);
      fa.head_sc = (m.lin_type == QT_LIN_Q8 || m.lin_type == QT_LIN_Q4) ? c->A<const uint16_t *>(c->L.f_heads_sc) : nullptr;
      fa.pos = c->A<int32_t>(c->L.pos); fa.c0 = c->A<int32_t>(c->L.c0); fa.bridge = c->A<float>(c->L.bridge);
      fa.ctl = c->A<int32_t>(c->L.ctl); fa.cin = c->A<int32_t>(c->L.cin); fa.cout = c->A<int32_t>(c->L.cout);
      fa.overlay = c->A<int32_t>(c->L.overlay);
      fa.rope_cos = c->A<float>(c->L.rope_cos); fa.rope_sin = c->A<float>(c->L.rope_sin);
      fa.ring_t = c->ring;
      fa.ring_p = c->ring + talker_ring_elems(d, c->B) * kv_elem(m);
      fa.t_kv_stride = (int64_t)d.kd * d.P; fa.t_layer_stride = 2 * fa.t_kv_stride;
      fa.p_kv_stride = (int64_t)d.kd * d.Q; fa.p_layer_stride = 2 * fa.p_kv_stride;
      fa.xq = c->A<uint64_t>(c->L.f_xq); fa.qkvb = c->A<uint64_t>(c->L.f_qkv);
      fa.ob = c->A<uint64_t>(c->L.f_o); fa.zb = c->A<uint64_t>(c->L.f_z);
      fa.amax = c->A<uint64_t>(c->L.f_amax); fa.part = c->A<uint64_t>(c->L.f_part);
      fa.lgx = c->A<uint64_t>(c->L.f_lgx);
      fa.logits_t = c->A<float>(c->L.logits_t); fa.logits_p = c->A<float>(c->L.logits_p);
      fa.x0_dump = c->A<float>(c->L.x0_dump); fa.hidden_dump = c->A<float>(c->L.hidden_dump);
      fa.gather_dump = c->A<int32_t>(c->L.gather_dump); fa.tpos_dump = c->A<int32_t>(c->L.tpos_dump);
      fa.dump = (c->flags & QT_F_DUMP) ? 1 : 0;
      fa.err = c->A<int32_t>(c->L.f_err);
      fa.trace = (c->flags & QT_F_TRACE) ? c->A<uint64_t>(c->L.f_trace) : nullptr;
      c->path = QT_PATH_FRAME;
      // the device address of this device's static exchange region, for
      // qt_decode_frame_noalloc (looked up here, once per device; a failure
      // only disables that entry point)
      if (qtk::frame_scratch_address(&c->scratch) != hipSuccess) c->scratch = nullptr;
    }
  }
  if (c->path == QT_PATH_GRAPH) {
    // the K-frame graph, and for K > 1 a 1-frame one (the tail of a call)
    for (int gi = 0; gi < (c->K > 1 ? 2 : 1); ++gi) {
      const int kf = gi == 0 ? c->K : 1;
      hipGraph_t &g = kf == c->K ? c->graph : c->graph1;
      hipGraphExec_t &x = kf == c->K ? c->exec : c->exec1;
      hipError_t e = hipStreamBeginCapture(c->stream, hipStreamCaptureModeRelaxed);
      if (e != hipSuccess) return bail(fail(c, QT_E_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e)));
      hipError_t eq = enqueue_replay(c, kf);
      e = hipStreamEndCapture(c->stream, &g);
      if (eq != hipSuccess) return bail(fail(c, QT_E_HIP, "frame capture: %s", hipGetErrorString(eq)));
      if (e != hipSuccess) return bail(fail(c, QT_E_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e)));
      e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
      if (e != hipSuccess) return bail(fail(c, QT_E_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e)));
    }
  }
  *out = c;
  return QT_OK;
}

int32_t qt_prefill(qt_ctx *c, int32_t slot, int32_t T, const int32_t *codes, const int32_t *text_ids) {
  return prefill_rows(c, 1, &slot, &T, codes, text_ids);
}

int32_t qt_prefill_rows(qt_ctx *c, int32_t n, const int32_t *slots, const int32_t *lengths, const int32_t *codes,
                        const int32_t *text_ids) {
  return prefill_rows(c, n, slots, lengths, codes, text_ids);
}

int32_t qt_decode_frame(qt_ctx *c, int32_t n, const int32_t *overlay_ids, int32_t *codes_out,
                        const int32_t *forced) {
  return decode_entry(c, n, overlay_ids, codes_out, forced, false);
}

int32_t qt_decode_frame_noalloc(qt_ctx *c, int32_t n, const int32_t *overlay_ids, int32_t *codes_out,
                                const int32_t *forced) {
  if (!c) return fail(nullptr, QT_E_ARG, "NULL context");
  if (c->path != QT_PATH_FRAME)
    return fail(c, QT_E_UNSUPPORTED, "qt_decode_frame_noalloc needs the persistent frame kernel (one stream)");
  const size_t need = c->L.f_err + 64 - c->L.f_xch_begin;
  if (need > qtk::kFrameScratchBytes)
    return fail(c, QT_E_SIZE, "the exchange region needs %zu bytes, above the static maximum of %zu", need,
                qtk::kFrameScratchBytes);
  if (!c->scratch) return fail(c, QT_E_HIP, "the static scratch address was not found at qt_init");
  return decode_entry(c, n, overlay_ids, codes_out, forced, true);
}

}  // extern "C"

namespace {

int32_t decode_entry(qt_ctx *c, int32_t n, const int32_t *overlay_ids, int32_t *codes_out, const int32_t *forced,
                     bool static_scratch) {
  if (!c) return fail(nullptr, QT_E_ARG, "NULL context");
  const Dims &d = c->d;
  const int B = c->B;
  if (n <= 0 || !overlay_ids || !codes_out) return fail(c, QT_E_ARG, "n_frames must be positive, pointers non-NULL");
  size_t short_rows = 0;  // paged: pool rows the new positions still need
  for (int b = 0; b < B; ++b) {
    if (!c->ready[b]) return fail(c, QT_E_STATE, "slot %d not prefilled", b);
    if (c->pos_host[b] + n > d.P)
      return fail(c, QT_E_CONTEXT_FULL, "slot %d: position %d + %d frames exceeds %d", b, c->pos_host[b], n, d.P);
    if (c->pool_rows) short_rows += rows_short(c, b, c->pos_host[b] + n);
  }
  if (short_rows > c->free_rows.size())
    return fail(c, QT_E_CONTEXT_FULL, "paged ring: %zu free rows, %d frames need %zu", c->free_rows.size(), n, short_rows);
  if (!ids_ok(overlay_ids, (size_t)n * B, d.Vt)) return fail(c, QT_E_RANGE, "overlay id outside [0, %d)", d.Vt);
  if (forced && !ids_ok(forced, (size_t)n * B * d.G, d.Vc)) return fail(c, QT_E_RANGE, "forced code outside [0, %d)", d.Vc);

  const int32_t rc = decode_chunks(c, n, overlay_ids, codes_out, forced, static_scratch);
  if (rc == QT_E_HIP)
    // work was launched: the slots may hold partial results (ring rows,
    // bridge, position), so they must be restored before the next decode
    for (int b = 0; b < B; ++b) c->ready[b] = 0;
  return rc;
}

int32_t prefill_rows(qt_ctx *c, int32_t n, const int32_t *slots, const int32_t *lens, const int32_t *codes,
                     const int32_t *text_ids) {
  if (!c) return fail(nullptr, QT_E_ARG, "NULL context");
  const Dims &d = c->d;
  if (n < 1 || n > PF_MAXROWS) return fail(c, QT_E_ARG, "streams per prefill call %d outside [1, %d]", n, PF_MAXROWS);
  if (!slots || !lens || !text_ids) return fail(c, QT_E_ARG, "NULL slots, lengths or text_ids");
  size_t total = 0, held = 0;
  for (int i = 0; i < n; ++i) {
    if (slots[i] < 0 || slots[i] >= c->B) return fail(c, QT_E_ARG, "slot %d outside [0, %d)", slots[i], c->B);
    for (int j = 0; j < i; ++j)
      if (slots[j] == slots[i]) return fail(c, QT_E_ARG, "slot %d given twice", slots[i]);
    if (lens[i] <= 0) return fail(c, QT_E_ARG, "prompt length %d must be positive", lens[i]);
    if (lens[i] > d.P) return fail(c, QT_E_CONTEXT_FULL, "prompt of %d rows exceeds %d ring positions", lens[i], d.P);
    total += (size_t)lens[i];
    if (c->pool_rows) held += c->slot_rows[slots[i]].size();
  }
  if (!ids_ok(text_ids, total, d.Vt)) return fail(c, QT_E_RANGE, "text id outside [0, %d)", d.Vt);
  if (codes && !ids_ok(codes, total * d.G, d.Vc)) return fail(c, QT_E_RANGE, "code id outside [0, %d)", d.Vc);
  if (c->pool_rows && c->free_rows.size() + held < total)
    return fail(c, QT_E_CONTEXT_FULL, "paged ring: %zu free rows, the prompts need %zu", c->free_rows.size() + held, total);

  // the chunks: positions [r0, r0 + t) of every stream still going
  struct Chunk {
    PfShape sh;
    int idoff, src[PF_MAXROWS], len[PF_MAXROWS], head[PF_MAXROWS];
  };
  std::vector<Chunk> plan;
  std::vector<size_t> first(n);  // each stream's first id row in text_ids
  for (int i = 0, acc = 0; i < n; acc += lens[i], ++i) first[i] = (size_t)acc;
  {
    std::vector<int> act(n);
    for (int i = 0; i < n; ++i) act[i] = i;
    int r0 = 0, idoff = 0;
    while (!act.empty()) {
      const int na = (int)act.size();
      int cap = kPrefillChunk;  // rows per stream so that na of them fit one chunk
      while (cap * na > kPrefillChunk) cap /= 2;
      int rem = 0;
      for (int i : act) rem = std::max(rem, lens[i] - r0);
      int t = kPfMinRows;
      while (t < rem && t < cap) t *= 2;
      if (r0 + t > d.P) t = d.P - r0;  // the ring's last positions
      Chunk ch = {};
      ch.sh.n = na; ch.sh.t = t; ch.sh.r0 = r0;
      ch.sh.tiles = std::min(c->L.max_tiles, (r0 + t - 1) / kTile + 1);
      ch.sh.codes = codes != nullptr;
      ch.idoff = idoff;
      for (int k = 0; k < na; ++k) {
        const int i = act[k];
        ch.src[k] = i;
        ch.len[k] = std::min(t, lens[i] - r0);
        ch.head[k] = lens[i] <= r0 + t ? k * t + ch.len[k] - 1 : -1;
        ch.sh.head = ch.sh.head || ch.head[k] >= 0;
      }
      plan.push_back(ch);
      idoff += na * t;
      r0 += t;
      act.erase(std::remove_if(act.begin(), act.end(), [&](int i) { return lens[i] <= r0; }), act.end());
    }
  }

  hipStream_t s = c->stream;
  const bool eager = c->flags & QT_F_EAGER;
  // every shape's graph is captured before this call's first copy, on the
  // idle stream (each earlier call ended with a synchronize)
  if (!eager)
    for (const Chunk &ch : plan) {
      if (c->pf_graphs.count(ch.sh.key()) || c->pf_graphs.size() >= kPfMaxGraphs) continue;
      hipGraph_t g = nullptr;
      hipGraphExec_t x = nullptr;
      HIPCHK(c, hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed));
      const hipError_t eq = enqueue_pf_chunk(c, ch.sh);
      const hipError_t ec = hipStreamEndCapture(s, &g);
      if (eq != hipSuccess || ec != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        return fail(c, QT_E_HIP, "prompt chunk capture: %s", hipGetErrorString(eq != hipSuccess ? eq : ec));
      }
      const hipError_t ei = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
      if (ei != hipSuccess) {
        (void)hipGraphDestroy(g);
        return fail(c, QT_E_HIP, "hipGraphInstantiate: %s", hipGetErrorString(ei));
      }
      c->pf_graphs[ch.sh.key()] = {g, x};
    }

  // from the first copy on the slots' ring rows change: they count as
  // prefilled again only once every chunk has run
  for (int i = 0; i < n; ++i) c->ready[slots[i]] = 0;
  // padded ids of every chunk, one upload
  int32_t *up_text = c->pin_up + c->pu_pf_text, *up_codes = c->pin_up + c->pu_pf_codes;
  size_t rows_total = 0;
  for (const Chunk &ch : plan) {
    for (int k = 0; k < ch.sh.n; ++k)
      for (int j = 0; j < ch.sh.t; ++j) {
        const size_t row = (size_t)ch.idoff + (size_t)k * ch.sh.t + j;
        const bool on = j < ch.len[k];
        const size_t src = first[ch.src[k]] + (size_t)(ch.sh.r0 + j);
        up_text[row] = on ? text_ids[src] : 0;
        if (codes)
          for (int g = 0; g < d.G; ++g) up_codes[row * d.G + g] = on ? codes[src * d.G + g] : 0;
      }
    rows_total = (size_t)ch.idoff + (size_t)ch.sh.n * ch.sh.t;
  }
  HIPCHK(c, hipMemcpyAsync(c->A<int32_t>(c->L.pf_text), up_text, sizeof(int32_t) * rows_total, hipMemcpyHostToDevice, s));
  if (codes)
    HIPCHK(c, hipMemcpyAsync(c->A<int32_t>(c->L.pf_codes), up_codes, sizeof(int32_t) * rows_total * d.G,
                             hipMemcpyHostToDevice, s));
  if (c->pool_rows) {  // the slots' rows back to the pool, then rows for their prompts
    for (int i = 0; i < n; ++i) release_slot(c, slots[i]);
    for (int i = 0; i < n; ++i) HIPCHK(c, grow_slot(c, slots[i], lens[i], c->pin_up + c->pu_ptab + (size_t)i * d.P));
  }
  for (size_t ci = 0; ci < plan.size(); ++ci) {
    const Chunk &ch = plan[ci];
    int32_t *w = c->pin_up + c->pu_pf_desc + ci * PF_WORDS;
    memset(w, 0, sizeof(int32_t) * PF_WORDS);
    w[PF_IDOFF] = ch.idoff;
    w[PF_R0] = ch.sh.r0;
    memcpy(&w[PF_ITEMP], &c->inv_temp, sizeof(float));
    w[PF_SEED_LO] = (int32_t)(uint32_t)c->seed;
    w[PF_SEED_HI] = (int32_t)(uint32_t)(c->seed >> 32);
    w[PF_TOPK] = c->top_k;
    for (int k = 0; k < ch.sh.n; ++k) {
      w[PF_SLOT + k] = slots[ch.src[k]];
      w[PF_LEN + k] = ch.len[k];
      w[PF_HEAD + k] = ch.head[k];
      w[PF_T + k] = lens[ch.src[k]];
    }
    HIPCHK(c, hipMemcpyAsync(c->A<int32_t>(c->L.pf_desc), w, sizeof(int32_t) * PF_WORDS, hipMemcpyHostToDevice, s));
    const auto gi = eager ? c->pf_graphs.end() : c->pf_graphs.find(ch.sh.key());
    if (gi == c->pf_graphs.end()) HIPCHK(c, enqueue_pf_chunk(c, ch.sh));
    else HIPCHK(c, hipGraphLaunch(gi->second.second, s));
  }
  HIPCHK(c, hipStreamSynchronize(s));
  for (int i = 0; i < n; ++i) {
    c->pos_host[slots[i]] = lens[i];
    c->ready[slots[i]] = 1;
  }
  return QT_OK;
}

int32_t decode_chunks(qt_ctx *c, int32_t n, const int32_t *overlay_ids, int32_t *codes_out,
                      const int32_t *forced, bool static_scratch) {
  const Dims &d = c->d;
  const int B = c->B;
  hipStream_t s = c->stream;
  int32_t *ctl = c->A<int32_t>(c->L.ctl);
  for (int f0 = 0; f0 < n; f0 += c->maxF) {
    const int nf = n - f0 < c->maxF ? n - f0 : c->maxF;
    // the previous chunk ended with a stream synchronize: staging is free
    int32_t *up = c->pin_up + c->pu_ctl;
    memset(up, 0, 16 * sizeof(int32_t));
    up[0] = 0;                 // frame index base
    up[1] = forced ? 1 : 0;    // teacher forcing
    memcpy(&up[2], &c->inv_temp, sizeof(float));  // sampler (argmax_kernel)
    up[3] = (int32_t)(uint32_t)c->seed;
    up[4] = (int32_t)(uint32_t)(c->seed >> 32);
    up[5] = c->top_k;
    int32_t *ov = c->pin_up + c->pu_overlay;
    memcpy(ov, overlay_ids + (size_t)f0 * B, sizeof(int32_t) * nf * B);
    HIPCHK(c, hipMemcpyAsync(ctl, up, 16 * sizeof(int32_t), hipMemcpyHostToDevice, s));
    HIPCHK(c, hipMemcpyAsync(c->A<int32_t>(c->L.overlay), ov, sizeof(int32_t) * nf * B, hipMemcpyHostToDevice, s));
    if (c->pool_rows)  // rows for the positions this chunk writes (counted by decode_entry)
      for (int b = 0; b < B; ++b)
        HIPCHK(c, grow_slot(c, b, c->pos_host[b] + nf, c->pin_up + c->pu_ptab + (size_t)b * c->maxF));
    if (forced) {
      int32_t *fu = c->pin_up + c->pu_forced;
      memcpy(fu, forced + (size_t)f0 * B * d.G, sizeof(int32_t) * nf * B * d.G);
      HIPCHK(c, hipMemcpyAsync(c->A<int32_t>(c->L.cin), fu, sizeof(int32_t) * nf * B * d.G, hipMemcpyHostToDevice, s));
    }
    qtk::FrameArgs fa = c->fa;
    if (c->path == QT_PATH_FRAME && static_scratch) {
      // The exchange words and the error flag live in this device's static
      // region, at their arena offsets.  Other contexts' calls leave their
      // own tags there, so the region is cleared first (tag 0 is never a
      // phase's tag): no word can match a tag of this launch before this
      // launch writes it.  (Calls that overlap on one device race.)
      uint8_t *base = (uint8_t *)c->scratch - c->L.f_xch_begin;
      fa.xq = (uint64_t *)(base + c->L.f_xq); fa.qkvb = (uint64_t *)(base + c->L.f_qkv);
      fa.ob = (uint64_t *)(base + c->L.f_o); fa.zb = (uint64_t *)(base + c->L.f_z);
      fa.amax = (uint64_t *)(base + c->L.f_amax); fa.part = (uint64_t *)(base + c->L.f_part);
      fa.lgx = (uint64_t *)(base + c->L.f_lgx);
      fa.err = (int32_t *)(base + c->L.f_err);
      HIPCHK(c, hipMemsetAsync(c->scratch, 0, c->L.f_err + 64 - c->L.f_xch_begin, s));
    } else if (c->path == QT_PATH_FRAME) {
      int32_t *zero = c->pin_up + c->pu_scalar + 4;
      zero[0] = 0;
      HIPCHK(c, hipMemcpyAsync(fa.err, zero, sizeof(int32_t), hipMemcpyHostToDevice, s));
    }
    if (c->path == QT_PATH_FRAME) {
      fa.n_frames = nf;
      fa.pos0 = c->pos_host[0];
      const char *why = nullptr;
      if (!qtk::frame_plan(fa, fa.pos0 + nf - 1, c->lds_limit, &why))
        return fail(c, QT_E_UNSUPPORTED, "frame kernel plan: %s", why);
      // Tags are only ever compared for equality, and each launch numbers
      // fewer than 1024 phases per frame.  When the 32-bit tag space would
      // wrap, every exchange word is cleared (tag 0, which no phase uses)
      // and numbering restarts: no word can then carry a tag of the coming
      // launch before that launch writes it.
      const uint64_t span = (uint64_t)nf * 1024u + 16u;
      if ((uint64_t)c->tag_base + span > 0xffffffffull) {
        HIPCHK(c, hipMemsetAsync(c->arena + c->L.f_xch_begin, 0, c->L.f_err - c->L.f_xch_begin, s));
        c->tag_base = 16u;
      }
      fa.tag_base = c->tag_base;
      fa.inv_temp = c->inv_temp;
      fa.seed = c->seed;
      fa.top_k = c->inv_temp != 0.f && c->top_k > 0 && c->top_k < d.Vc ? c->top_k : 0;
      c->tag_base += (uint32_t)span;
      HIPCHK(c, launch_frame_kernel(fa, s));
    } else {
      // adaptive K: whole K-frame blocks, then the rest one frame at a time
      for (int r = 0; r < nf / c->K; ++r) {
        if (c->exec) HIPCHK(c, hipGraphLaunch(c->exec, s));
        else HIPCHK(c, enqueue_replay(c, c->K));
      }
      for (int r = 0; r < nf % c->K; ++r) {
        if (c->exec1) HIPCHK(c, hipGraphLaunch(c->exec1, s));
        else HIPCHK(c, enqueue_replay(c, 1));
      }
    }
    HIPCHK(c, hipMemcpyAsync(c->pin_down, c->A<int32_t>(c->L.cout), sizeof(int32_t) * nf * B * d.G, hipMemcpyDeviceToHost, s));
    int32_t *errh = c->pin_up + c->pu_scalar + 8;
    errh[0] = 0;
    if (c->path == QT_PATH_FRAME)
      HIPCHK(c, hipMemcpyAsync(errh, fa.err, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    HIPCHK(c, hipStreamSynchronize(s));
    if (errh[0])
      return fail(c, QT_E_HIP, "frame kernel: an exchange wait timed out (the slot must be restored by "
                                "qt_prefill or qt_set_slot_state)");
    memcpy(codes_out + (size_t)f0 * B * d.G, c->pin_down, sizeof(int32_t) * nf * B * d.G);
    for (int b = 0; b < B; ++b) c->pos_host[b] += nf;
  }
  return QT_OK;
}

}  // namespace

extern "C" {

int32_t qt_get_slot_state(qt_ctx *c, int32_t slot, int32_t *pos, int32_t *c0, float *bridge) {
  if (!c) return fail(nullptr, QT_E_ARG, "NULL context");
  if (slot < 0 || slot >= c->B) return fail(c, QT_E_ARG, "slot %d outside [0, %d)", slot, c->B);
  HIPCHK(c, hipStreamSynchronize(c->stream));
  if (pos) HIPCHK(c, hipMemcpy(pos, c->A<int32_t>(c->L.pos) + slot, 4, hipMemcpyDeviceToHost));
  if (c0) HIPCHK(c, hipMemcpy(c0, c->A<int32_t>(c->L.c0) + slot, 4, hipMemcpyDeviceToHost));
  if (bridge)
    HIPCHK(c, hipMemcpy(bridge, c->A<float>(c->L.bridge) + (size_t)slot * c->d.H, sizeof(float) * c->d.H, hipMemcpyDeviceToHost));
  return QT_OK;
}

int32_t qt_set_slot_state(qt_ctx *c, int32_t slot, int32_t pos, int32_t c0, const float *bridge) {
  if (!c) return fail(nullptr, QT_E_ARG, "NULL context");
  if (slot < 0 || slot >= c->B || !bridge) return fail(c, QT_E_ARG, "bad slot or NULL bridge");
  if (pos < 1 || pos > c->d.P) return fail(c, QT_E_RANGE, "pos %d outside [1, %d]", pos, c->d.P);
  if (c0 < 0 || c0 >= c->d.Vc) return fail(c, QT_E_RANGE, "c0 %d outside [0, %d)", c0, c->d.Vc);
  if (c->pool_rows && c->slot_rows[slot].size() < (size_t)pos)
    return fail(c, QT_E_STATE, "paged ring: slot %d holds %zu rows, pos %d needs them all", slot, c->slot_rows[slot].size(), pos);
  c->ready[slot] = 0;  // until every part of the state is written
  HIPCHK(c, hipStreamSynchronize(c->stream));
  HIPCHK(c, hipMemcpy(c->A<int32_t>(c->L.pos) + slot, &pos, 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->A<int32_t>(c->L.c0) + slot, &c0, 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->A<float>(c->L.bridge) + (size_t)slot * c->d.H, bridge, sizeof(float) * c->d.H, hipMemcpyHostToDevice));
  c->pos_host[slot] = pos;
  c->ready[slot] = 1;
  return QT_OK;
}

int32_t qt_read_dump(qt_ctx *c, int32_t kind, void *dst, size_t bytes) {
  if (!c) return fail(nullptr, QT_E_ARG, "NULL context");
  if (kind == QT_DUMP_TRACE ? !(c->flags & QT_F_TRACE) : !(c->flags & QT_F_DUMP))
    return fail(c, QT_E_STATE, "dump %d needs QT_F_DUMP (QT_F_TRACE for the trace)", kind);
  if (!dst) return fail(c, QT_E_ARG, "NULL destination");
  const Dims &d = c->d;
  const size_t B = c->B;
  size_t off, need;
  switch (kind) {
    case QT_DUMP_TALKER_LOGITS: off = c->L.logits_t; need = 4 * B * d.Vc; break;
    case QT_DUMP_PRED_LOGITS: off = c->L.logits_p; need = 4 * (size_t)(d.G - 1) * B * d.Vc; break;
    case QT_DUMP_BRIDGE: off = c->L.bridge; need = 4 * B * d.H; break;
    case QT_DUMP_X0: off = c->L.x0_dump; need = 4 * B * d.H; break;
    case QT_DUMP_GATHER: off = c->L.gather_dump; need = 4 * B * (d.G + 1); break;
    case QT_DUMP_TPOS: off = c->L.tpos_dump; need = 4 * B; break;
    case QT_DUMP_HIDDEN: off = c->L.hidden_dump; need = 4 * (size_t)d.Lt * B * d.H; break;
    case QT_DUMP_TRACE: off = c->L.f_trace; need = 8 * 8 * 1024; break;
    default: return fail(c, QT_E_ARG, "unknown dump kind %d", kind);
  }
  if (bytes != need) return fail(c, QT_E_ARG, "dump %d is %zu bytes, not %zu", kind, need, bytes);
  HIPCHK(c, hipStreamSynchronize(c->stream));
  HIPCHK(c, hipMemcpy(dst, c->arena + off, need, hipMemcpyDeviceToHost));
  return QT_OK;
}

int32_t qt_time_kernel(qt_ctx *c, int32_t kernel, int32_t reps, double *avg_us, double *bytes) {
  if (!c) return fail(nullptr, QT_E_ARG, "NULL context");
  if (kernel != QT_KERNEL_GEMV_GATE_UP || reps <= 0 || !avg_us || !bytes)
    return fail(c, QT_E_ARG, "unknown kernel or bad arguments");
  const Dims &d = c->d;
  const qt_model_desc &md = c->md;
  const int wt = wtype_of(md);
  hipStream_t s = c->stream;
  hipEvent_t e0, e1;
  HIPCHK(c, hipEventCreate(&e0));
  HIPCHK(c, hipEventCreate(&e1));
  std::vector<const qt_layer_weights *> layers;
  for (auto &L : c->tl) layers.push_back(&L);
  for (auto &L : c->pl) layers.push_back(&L);
  GemvArgs gu = {};
  gu.act_bf16 = md.act_bf16; gu.gain_bf16 = md.tab_bf16; gu.eps = (float)md.eps;
  gu.nseg = 1; gu.seg_end[0] = d.F; gu.N = d.F; gu.K = d.H;
  gu.x = c->A<float>(c->L.x); gu.x_stride = d.H; gu.M = c->B;
  gu.y = c->A<float>(c->L.z); gu.y_stride = d.F;
  // as the per-op decode path runs it (project(): the split-K MFMA GEMM for
  // bf16, q8 and q4 models whose widths are multiples of 256, at 1..512 rows,
  // its row norms reading the sums of squares the last decode left; else the
  // GEMV)
  (void)wt;
  hipError_t err = hipEventRecord(e0, s);
  int launches = 0;
  for (int r = 0; r < reps && err == hipSuccess; ++r)
    for (const qt_layer_weights *L : layers) {
      gu.seg[0] = lin(L->wg); gu.up = lin(L->wu); gu.gain = L->mlp_norm;
      if ((err = project(c, EPI_GATED, gu, c->A<float>(c->L.ssq), d.H / 32, nullptr)) != hipSuccess) break;
      ++launches;
    }
  if (err == hipSuccess) err = hipEventRecord(e1, s);
  if (err == hipSuccess) err = hipEventSynchronize(e1);
  float ms = 0.f;
  if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err != hipSuccess) return fail(c, QT_E_HIP, "qt_time_kernel: %s", hipGetErrorString(err));
  const double wbytes = md.lin_type == QT_LIN_F32 ? 4.0 : md.lin_type == QT_LIN_BF16 ? 2.0
                        : md.lin_type == QT_LIN_Q8 ? 34.0 / 32.0 : 18.0 / 32.0;
  *avg_us = 1000.0 * ms / launches;
  *bytes = 2.0 * d.F * d.H * wbytes + 4.0 * c->B * (d.H + d.F);
  return QT_OK;
}

int32_t qt_stream_read(const void *src, size_t bytes, void *sink, size_t sink_bytes, int32_t reps, void *stream,
                       double *avg_us) {
  if (!src || !sink || !avg_us || reps <= 0) return fail(nullptr, QT_E_ARG, "NULL pointer or reps <= 0");
  if (bytes < (1u << 20) || bytes % 16 || ((uintptr_t)src | (uintptr_t)sink) % 16)
    return fail(nullptr, QT_E_ARG, "bytes must be >= 1 MiB and a multiple of 16; pointers 16-byte aligned");
  if (sink_bytes < (size_t)kStreamGrid * 256 * 4)
    return fail(nullptr, QT_E_SIZE, "sink needs %zu bytes", (size_t)kStreamGrid * 256 * 4);
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return fail(nullptr, QT_E_HIP, "hipEventCreate failed");
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return fail(nullptr, QT_E_HIP, "hipEventCreate failed");
  }
  hipError_t err = launch_stream_read(src, bytes, sink, s);  // untimed first pass
  if (err == hipSuccess) err = hipEventRecord(e0, s);
  for (int r = 0; r < reps && err == hipSuccess; ++r) err = launch_stream_read(src, bytes, sink, s);
  if (err == hipSuccess) err = hipEventRecord(e1, s);
  if (err == hipSuccess) err = hipEventSynchronize(e1);
  float ms = 0.f;
  if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err != hipSuccess) return fail(nullptr, QT_E_HIP, "qt_stream_read: %s", hipGetErrorString(err));
  *avg_us = 1000.0 * ms / reps;
  return QT_OK;
}

}  // extern "C"
