// frame.h -- the persistent frame kernel (internal to libqt).
//
// One launch decodes n frames of one stream.  Every workgroup walks the same
// phase schedule (15 code-predictor micro-steps of Lp layers, then the talker
// step of Lt layers, per frame).  The first n_attn workgroups run attention
// only (one KV head and one tile of talker positions each, with that tile's
// K/V held in LDS); the others run every projection, MLP and head as
// weight-streaming GEMVs.  Phases hand data to each other through tagged
// 64-bit words (tag | value) stored and loaded at agent scope.
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

struct FrameArgs {
  // shapes
  int32_t H, nq, nkv, hd, F, Lt, Lp, G, Vc, Vt, P, Q;
  int32_t wt, tab_bf16, kv_bf16, act_bf16;
  float eps, scale;
  // launch plan (frame_plan)
  int32_t nwg;         // workgroups, one per compute unit
  int32_t n_attn;      // leading attention workgroups: kv head = wg % nkv, tile = wg / nkv
  int32_t tile;        // talker positions per attention tile
  int32_t max_tiles;   // tiles per head in the partial buffer
  int32_t slot_bytes;  // LDS bytes of one weight slot
  int32_t two_slots;   // 1: the next phase's weights stream in while this phase computes
  int32_t lds_bytes;   // dynamic LDS per workgroup
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
  // tagged exchange words
  uint64_t *xq;    // [2][H]        residual stream rows
  uint64_t *qkvb;  // [2][nqkv]     q | k | v rows
  uint64_t *ob;    // [2][nq*hd]    attention output (bf16 pairs when act_bf16)
  uint64_t *zb;    // [2][F]        SiLU-mul output (bf16 pairs when act_bf16)
  uint64_t *amax;  // [nwg][2]      per-workgroup (value, index) of a head's argmax
  uint64_t *part;  // [nq][max_tiles][hd + 2]  tile partials (o, max, sum)
  // xq, ob and zb exist rep times, rep_stride words apart: producers write
  // every copy, workgroup b reads copy b % rep, so that the readers of one
  // row spread over rep places in memory
  int32_t rep;
  int64_t rep_stride;
  // outputs / dumps
  float *logits_t;  // [Vc]
  float *logits_p;  // [G-1][Vc]
  float *x0_dump, *hidden_dump;  // [H], [Lt][H]
  int32_t *gather_dump, *tpos_dump;
  int32_t dump;
  // control
  int32_t pos0;       // talker position of the launch's first frame (the slot's position)
  int32_t n_frames;
  uint32_t tag_base;  // tags of this launch are tag_base + phase index (> 0)
  int32_t *err;       // [0] set on a timed-out wait
  uint64_t *trace;    // optional: [1024][8] stamps (rows < 768: first GEMV workgroup; rest: attention workgroup 0)
  float inv_temp;     // sampling (sampler.h): float(1/T), 0 = greedy
  uint64_t seed;
  int32_t top_k;      // sampling: only the top_k largest logits compete (0: all; Vc <= 2048)
  uint64_t *lgx;      // [Vc] tagged head logits, for top_k > 0
};

// Cooperative launch: every workgroup is resident at once, or the launch fails.
hipError_t launch_frame_kernel(const FrameArgs &a, hipStream_t s);
// True if a.nwg workgroups of the planned kernel (a.lds_bytes of LDS each)
// fit on the ncu compute units at once, by the occupancy query.
bool frame_coresident(const FrameArgs &a, int ncu);
// Device address of this device's static scratch array (kFrameScratchBytes),
// looked up once per device with that device current.
constexpr size_t kFrameScratchBytes = 512u << 10;
constexpr int kMaxDevices = 64;
hipError_t frame_scratch_address(void **ptr);
// the (weights, head dim, GQA group, bf16 ring) combinations instantiated
bool frame_variant_supported(int wt, int hd, int g, int kv_bf16);
// Plan a launch whose talker positions reach max_pos: attention workgroups,
// tile, weight slots and LDS size.  False (with *why) if it does not fit.
bool frame_plan(FrameArgs &a, int max_pos, int lds_limit, const char **why);

}  // namespace qtk
