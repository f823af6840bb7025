// frame.h -- the persistent frame kernel (internal to libqt).
//
// One launch decodes n frames for one stream: every workgroup walks the same
// phase schedule (15 code-predictor micro-steps of Lp layers, then the talker
// step of Lt layers, per frame).  Phases hand data to each other through
// tagged 64-bit words (tag | value) stored and loaded at agent scope, so a
// consumer waits on the data itself; each workgroup keeps the next phase's
// weight slice in flight in registers while it waits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qtk {

struct LayerDev {
  const void *attn_norm, *q_norm, *k_norm, *mlp_norm;
  const void *w[7];       // wq, wk, wv, wo, wg, wu, wd
  const uint16_t *sc[7];  // q8 scales (fp16 bits) or null
};
enum { LW_Q = 0, LW_K, LW_V, LW_O, LW_G, LW_U, LW_D };

// GEMV work split of one phase kind: output rows per wave, weight matrices per
// output row (2 for gate/up), 16-byte chunks per lane per weight row.
struct Split {
  int8_t rw, nmat, cpl;
};
enum { SP_QKV = 0, SP_O, SP_GU, SP_D, SP_HEAD, SP_COUNT };

struct FrameArgs {
  // shapes
  int32_t H, nq, nkv, hd, F, Lt, Lp, G, Vc, Vt, P, Q;
  int32_t wt, tab_bf16, kv_bf16, act_bf16;
  float eps, scale;
  Split split[SP_COUNT];
  int32_t nwg;
  // weights
  const LayerDev *tl, *pl;                  // device arrays [Lt], [Lp]
  const void *code_emb, *text_emb, *t_norm, *p_norm;
  const void *const *head_w;                // device array [G]: 0 talker, 1..G-1 predictor
  const uint16_t *const *head_sc;           // device array [G] (q8) or null
  // slot state (slot 0)
  int32_t *pos, *c0;
  float *bridge;
  const int32_t *ctl;                       // [0] frame base (0), [1] teacher forcing
  int32_t *cin, *cout;                      // [frames][1][G]
  const int32_t *overlay;                   // [frames][1]
  const float *rope_cos, *rope_sin;         // [P][hd/2]
  uint8_t *ring_t, *ring_p;                 // (slot 0, layer 0, K) of each stack
  int64_t t_layer_stride, t_kv_stride, p_layer_stride, p_kv_stride;  // elements
  // tagged exchange buffers
  uint64_t *xq;    // [2][H]
  uint64_t *qkvb;  // [2][nqkv]
  uint64_t *ob;    // [2][nq*hd]
  uint64_t *zb;    // [2][F]
  uint64_t *amax;  // [nwg][2]  (value | index) per workgroup
  uint64_t *part;  // [nq][P/256][hd + 2]
  // outputs / dumps
  float *logits_t;  // [Vc]
  float *logits_p;  // [G-1][Vc]
  float *x0_dump, *hidden_dump;  // [H], [Lt][H]
  int32_t *gather_dump, *tpos_dump;
  int32_t dump;
  // control
  int32_t n_frames;
  uint32_t tag_base;  // tags of this launch are tag_base + phase index (> 0)
  int32_t *err;     // [0] set on a timed-out wait
  uint64_t *trace;  // optional: [1024][8] phase stamps of workgroup 0, first frame
};

hipError_t launch_frame_kernel(const FrameArgs &a, hipStream_t s);
// the (rows/wave, matrices, chunks/lane) triples the kernel is instantiated for
bool frame_split_supported(int wt, const Split &sp);
// the (weights, head dim, GQA group, bf16 ring) combinations instantiated
bool frame_variant_supported(int wt, int hd, int g, int kv_bf16);
// LDS the kernel needs per workgroup (dynamic shared memory)
size_t frame_lds_bytes();

}  // namespace qtk
