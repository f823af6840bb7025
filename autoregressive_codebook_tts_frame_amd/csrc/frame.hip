// frame.hip -- persistent frame kernel for one stream (gfx950, wave64).
//
// The frame is a chain of dependent phases: per code-predictor micro-step
// ([QT-log] per-layer K/V ring entry: a 2-row prefill then 14 single-row
// decodes) and per talker step, each layer is QKV -> attention -> O (+residual)
// -> gate/up (+SiLU-mul) -> down (+residual), then a head whose argmax picks
// the next code ([QT-tests] fused codec mode entry: in-graph sampler).  A
// kernel launch per phase costs more than the phase's own HBM traffic (the
// failure mode [MC-opt] reports in its closing paragraph), so one launch runs
// every phase of n frames.  At batch 1 each phase is one exchange of a few KB
// between all compute units, so the design works on exchange latency first:
//
//  * Two roles.  The first n_attn workgroups only run attention: workgroup
//    (KV head kh, tile t) keeps the K/V rows of talker positions
//    [256 t, 256 t + 256) of the layer it serves next in LDS (streamed in from
//    the ring while the GEMV phases run) and, for t = 0, the 16-position
//    code-predictor cache of its head.  The other workgroups run every
//    projection, the MLP and the heads as GEMVs over their rows.
//  * One exchange per phase.  A phase's outputs are 64-bit words
//    (tag | value) stored at agent scope; a consumer loads all the words it
//    needs at once and retries only those whose tag is not yet the producing
//    phase's.  Every wait is bounded: a timed-out wait raises a device error
//    flag and the kernel drains.
//  * Weights stream through LDS.  Right after a GEMV workgroup has its
//    inputs it issues direct-to-LDS loads of the next GEMV phase's weight
//    slice (and norm gain) into the other of two slots, so the HBM stream
//    overlaps this phase's compute and the next exchange.  These loads are
//    issued from inline assembly: vector-memory counters complete in order,
//    and the only waits on them are the exchange waits that follow.
//  * Residuals and gathers stay local.  Each GEMV workgroup keeps the last
//    residual row it read in LDS (the O and down epilogues add to it) and
//    accumulates the talker's gather-sum ([QT-log] AR inputs entry) in
//    registers as the predictor picks each code, in code order.
#include <math.h>

#include <mutex>

#include "frame.h"
#include "kernels.h"
#include "sampler.h"

namespace qtk {
namespace {

constexpr int NW = 5;            // compute waves of a GEMV workgroup
constexpr int NT = 64 * NW;      // their threads
constexpr int NLW = 3;           // loader waves (each keeps its own loads in flight)
constexpr int TKU = 7;           // top-k: logits per compute thread (Vc <= 2048 = 7 * 320 - 192)
constexpr int NTB = NT + 64 * NLW;  // two waves per SIMD
constexpr int ANT = 512;         // threads of an attention workgroup
constexpr int ANW = ANT / 64;    // its waves
constexpr int MAXLAYERS = 40;
constexpr int MAXHEADS = 32;
constexpr int PER = 8;          // tagged words per thread per poll round
constexpr int HPAIR = 3;        // hidden pairs per thread (H <= 2 * NT * HPAIR)
constexpr int MAXR = 64;        // GEMV rows per workgroup per phase
constexpr int TILE = 256;       // talker positions per attention tile
constexpr uint32_t SPIN_LIMIT = 1u << 21;

enum { PH_QKV = 0, PH_ATTN, PH_COMB, PH_O, PH_GU, PH_D, PH_HEAD, PH_END };

struct Ph {
  int type, stack, layer, step, frame;  // stack 0 predictor, 1 talker; step = micro-step
};

// Every global access goes through a global-address-space pointer: flat
// accesses would also count against the LDS wait counter.
#define GAS __attribute__((address_space(1)))
#define LAS __attribute__((address_space(3)))
template <class T> __device__ __forceinline__ GAS T *gp(T *p) { return (GAS T *)p; }
template <class T> __device__ __forceinline__ const GAS T *gp(const T *p) { return (const GAS T *)p; }

// float -> nearest bf16 (ties to even; the hardware conversion), kept in a float
__device__ __forceinline__ float bf16_rne(float f) {
  return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f) << 16);
}
__device__ __forceinline__ uint32_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// nearest bf16 pair of (lo, hi), lo in the low half: one packed conversion
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
// Cross-lane reductions with DPP row operations (a row is 16 lanes) and
// readlane for the four row results: a few VALU cycles per step, where a
// shuffle chain would go through the LDS crossbar once per step.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float row16_sum(float v) {  // every lane gets its row's sum
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x128>(v));
  return v;
}
__device__ __forceinline__ float lane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
__device__ __forceinline__ float wave_sum(float v) {  // uniform result
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
// greedy pick: larger value wins, the lower index on ties
__device__ __forceinline__ void pick(float &bv, int &bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}
template <int CTRL>
__device__ __forceinline__ void pick_dpp(float &bv, int &bi) {
  pick(bv, bi, dpp<CTRL>(bv), __builtin_amdgcn_update_dpp(0, bi, CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ void wave_argmax(float &bv, int &bi) {  // uniform result
  pick_dpp<0xB1>(bv, bi);
  pick_dpp<0x4E>(bv, bi);
  pick_dpp<0x124>(bv, bi);
  pick_dpp<0x128>(bv, bi);
  float v = lane_f(bv, 0);
  int i = __builtin_amdgcn_readlane(bi, 0);
  pick(v, i, lane_f(bv, 16), __builtin_amdgcn_readlane(bi, 16));
  pick(v, i, lane_f(bv, 32), __builtin_amdgcn_readlane(bi, 32));
  pick(v, i, lane_f(bv, 48), __builtin_amdgcn_readlane(bi, 48));
  bv = v;
  bi = i;
}

template <class T> __device__ __forceinline__ T ld(const T *p) { return *gp(p); }
template <class T> __device__ __forceinline__ void st(T *p, T v) { *gp(p) = v; }

// tagged words: tags run on across launches (tag_base advances per launch)
__device__ __forceinline__ void tput(uint64_t *p, uint32_t v, uint32_t tag) {
  __hip_atomic_store(gp(p), ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void tputf(uint64_t *p, float v, uint32_t tag) { tput(p, __float_as_uint(v), tag); }
__device__ __forceinline__ uint64_t tget(const uint64_t *p) {
  return __hip_atomic_load(gp(const_cast<uint64_t *>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int err_get(const int32_t *e) {
  return __hip_atomic_load(gp(const_cast<int32_t *>(e)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void err_set(int32_t *e) {
  __hip_atomic_store(gp(e), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// ring rows: 8-byte words at agent scope, so the tile loads below (which
// bypass the caches the same way) see them
__device__ __forceinline__ void ring_put(uint8_t *p, uint64_t v) {
  __hip_atomic_store(gp((uint64_t *)p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One 16-byte-per-lane direct-to-LDS load: lane l's bytes land at
// lds_base + 16 l.  coherent: load at agent scope (ring rows).
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(src)
      : "memory");
}
__device__ __forceinline__ void dma16_coherent(const void *src, uint32_t lds_base) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off sc1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(src)
      : "memory");
}
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const LAS void *)p;
}

// Weight pointers of every layer and head, copied into LDS at kernel start.
struct LayerTab {
  const void *w[7];
  const uint16_t *sc[7];
  const void *attn_norm, *q_norm, *k_norm, *mlp_norm;
};

// GEMV rows [r0, r0 + R) of N, width K, NM matrices (2: gate and up)
struct Share {
  int r0, R, N, K, NM;
};

struct Common {
  LayerTab lt[MAXLAYERS];  // talker layers then predictor layers
  const void *head_w[MAXHEADS];
  const uint16_t *head_sc[MAXHEADS];
  float amv[NW];
  int ami[NW];
  float pss[2][NW];     // per-wave partial sums of squares of the residual rows
  int codes[MAXHEADS];  // codes fed to this frame's gathers
  int code;
  int abort;
  uint32_t cbar;   // compute-wave barrier arrivals
  uint32_t gdone;  // GEMV completions (compute waves; loader waves where they take items)
  uint32_t hist[256];       // top-k: radix-select histogram
  uint32_t tsel[2];         // top-k: the threshold key and the last member's index
  uint64_t ltime;  // tracing: when a loader wave's part of the last slice had landed
  Share sh[PH_END];  // this GEMV workgroup's rows, per phase type
};

// Offsets (bytes) of each role's LDS buffers; one function for host and device.
struct Lds {
  uint32_t xres, opnd, res, brg, tacc, slot0, slot1, g_end;            // GEMV role
  uint32_t gq, gk, rc, rs, rowbuf, sc, stat, pvred, comb, kv, a_end;    // attention role
};
__host__ __device__ inline uint32_t up16(uint32_t v) { return (v + 15u) & ~15u; }
__host__ __device__ inline uint32_t up1k(uint32_t v) { return (v + 1023u) & ~1023u; }
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ inline Lds lds_layout(const FrameArgs &a) {
  Lds L;
  const uint32_t base = up16(sizeof(Common));
  // GEMV role
  const int kop = imax(a.H, imax(a.nq * a.hd, a.F));
  const int opw = imax(imax(a.act_bf16 ? kop / 2 : kop, 2 * a.nwg), (a.Vc + 1) / 2);
  L.xres = base;
  L.opnd = up16(L.xres + 2u * a.H * 4u);
  L.res = up16(L.opnd + 2u * opw * 4u);
  L.brg = up16(L.res + MAXR * 4u * 4u);
  L.tacc = L.brg + a.H * 4u;
  L.slot0 = up1k(L.tacc + a.H * 4u);
  L.slot1 = L.slot0 + (a.two_slots ? (uint32_t)a.slot_bytes : 0u);
  L.g_end = L.slot1 + a.slot_bytes;
  // attention role (G query heads per KV head)
  const int g = a.nq / a.nkv, hd = a.hd;
  const uint32_t rowb = (uint32_t)hd * (a.kv_bf16 ? 2u : 4u);
  L.gq = base;
  L.gk = L.gq + hd * 4u;
  L.rc = L.gk + hd * 4u;
  L.rs = L.rc + hd * 4u;  // [2][hd/2] each
  // attention scratch and the tile-merge buffer are never live together
  L.rowbuf = up16(L.rs + hd * 4u);
  L.sc = up16(L.rowbuf + 2u * (g + 2) * hd * 4u);
  L.stat = up16(L.sc + (uint32_t)g * a.tile * 4u);
  L.pvred = up16(L.stat + 4u * g * 4u);
  L.comb = L.rowbuf;
  const uint32_t scratch_end = up16(L.pvred + (uint32_t)ANW * g * hd * 4u);
  const uint32_t comb_end = L.comb + (uint32_t)g * a.max_tiles * (hd + 2) * 4u;
  L.kv = up1k(scratch_end > comb_end ? scratch_end : comb_end);
  const uint32_t tile_b = 2u * a.tile * rowb, pc_b = (uint32_t)a.Lp * 2u * a.Q * rowb;
  L.a_end = L.kv + up1k(tile_b > pc_b ? tile_b : pc_b);
  return L;
}

// ------------------------------------------------------------ schedule

__device__ __forceinline__ int ntiles_at(int p) { return p / TILE + 1; }

__device__ __forceinline__ Ph next_phase(const FrameArgs &a, const Ph &p, int pos0) {
  Ph n = p;
  switch (p.type) {
    case PH_QKV: n.type = PH_ATTN; break;
    case PH_ATTN: n.type = (p.stack == 1 && ntiles_at(pos0 + p.frame) > 1) ? PH_COMB : PH_O; break;
    case PH_COMB: n.type = PH_O; break;
    case PH_O: n.type = PH_GU; break;
    case PH_GU: n.type = PH_D; break;
    case PH_D:
      if (p.layer + 1 < (p.stack ? a.Lt : a.Lp)) { n.type = PH_QKV; n.layer = p.layer + 1; }
      else n.type = PH_HEAD;
      break;
    case PH_HEAD:
      n.layer = 0;
      n.type = PH_QKV;
      if (p.stack == 0) {
        if (p.step + 1 < a.G - 1) n.step = p.step + 1;
        else { n.stack = 1; n.step = 0; }
      } else {
        n.stack = 0; n.step = 0; n.frame = p.frame + 1;
        if (n.frame >= a.n_frames) n.type = PH_END;
      }
      break;
    default: n.type = PH_END;
  }
  return n;
}
__device__ __forceinline__ Ph next_gemv_phase(const FrameArgs &a, Ph p, int pos0) {
  do p = next_phase(a, p, pos0);
  while (p.type == PH_ATTN || p.type == PH_COMB);
  return p;
}
__device__ __forceinline__ const LayerTab &tab_of(const FrameArgs &a, const Common &cm, int stack, int layer) {
  return cm.lt[stack ? layer : a.Lt + layer];
}

// ------------------------------------------------------------ exchange

// Poll n tagged words (word i at src(i)) until each carries tag; value bits
// -> *dst(i) (LDS).  All threads; false on timeout.
struct NoTap {
  __device__ __forceinline__ void operator()(int, uint32_t) const {}
};
// Wait for n tagged words src(i) and store their values at dst(i); every
// value also goes to tap(i, v), in this thread's order.
template <int TH = NT, class Dst, class Src, class Tap = NoTap>
__device__ __forceinline__ bool poll(const FrameArgs &a, int n, uint32_t tag, Dst dst, Src src, Tap tap = Tap()) {
  for (int b0 = 0; b0 < n; b0 += PER * TH) {
    uint64_t v[PER];
    uint32_t pend = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = b0 + (int)threadIdx.x + k * TH;
      if (i < n) { v[k] = tget(src(i)); pend |= 1u << k; }
    }
    for (uint32_t spins = 0;; ++spins) {
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if (((pend >> k) & 1u) && (uint32_t)(v[k] >> 32) == tag) {
          *dst(b0 + threadIdx.x + k * TH) = (uint32_t)v[k];
          tap(b0 + threadIdx.x + k * TH, (uint32_t)v[k]);
          pend &= ~(1u << k);
        }
      if (!pend) {
        // Nothing is in flight now, but the compiler cannot see it: without
        // this it waits for all memory operations before every later write
        // to these registers, serialising the next poll's loads.
        wait_vm();
        break;
      }
      if (spins > SPIN_LIMIT || ((spins & 255u) == 255u && err_get(a.err))) {
        err_set(a.err);
        wait_vm();  // leave no load in flight into registers the caller reuses
        return false;
      }
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if ((pend >> k) & 1u) v[k] = tget(src(b0 + threadIdx.x + k * TH));
    }
  }
  return true;
}
template <int TH = NT, class Tap = NoTap>
__device__ __forceinline__ bool poll_lin(const FrameArgs &a, const uint64_t *src, int n, uint32_t tag, uint32_t *dst,
                                         Tap tap = Tap()) {
  return poll<TH>(a, n, tag, [=](int i) { return dst + i; }, [=](int i) { return src + i; }, tap);
}
// one or two rows of w words at src (contiguous) into LDS rows of stride dw
template <class Tap = NoTap>
__device__ __forceinline__ bool poll_rows(const FrameArgs &a, const uint64_t *src, int rows, int w, uint32_t tag,
                                          uint32_t *dst, int dw, Tap tap = Tap()) {
  return poll(a, rows * w, tag, [=](int i) { return dst + (i < w ? i : i - w + dw); },
              [=](int i) { return src + i; }, tap);
}

// ------------------------------------------------------------ GEMV role

// Rows of phase type `type`: count N, width K, NM matrices (2: gate and up).
__device__ __forceinline__ Share shape_of(const FrameArgs &a, int type) {
  Share s;
  const int qd = a.nq * a.hd;
  s.NM = 1;
  switch (type) {
    case PH_QKV: s.N = qd + 2 * a.nkv * a.hd; s.K = a.H; break;
    case PH_O: s.N = a.H; s.K = qd; break;
    case PH_GU: s.N = a.F; s.K = a.H; s.NM = 2; break;
    case PH_D: s.N = a.H; s.K = a.F; break;
    default: s.N = a.Vc; s.K = a.H; break;
  }
  return s;
}
// Row share of GEMV workgroup gi among NG: rows [r0, r0 + R), computed once
// per phase type at the start, then read from LDS.  Gate/up rows go in pairs
// (one packed bf16 pair of SiLU-mul outputs each), the others one by one, so
// no workgroup gets more than one unit above the mean.  The workgroups that
// get that extra unit are dealt round-robin across the phase types in their
// order within a layer: a workgroup with an extra row in every phase type
// would fall further behind each phase and pace the whole frame.
__device__ __forceinline__ Share share_calc(const FrameArgs &a, int type, int gi, int NG) {
  Share s = shape_of(a, type);
  const int order[5] = {PH_QKV, PH_O, PH_GU, PH_D, PH_HEAD};
  int off = 0;  // extra units dealt to the phase types before this one
  for (int k = 0; k < 5 && order[k] != type; ++k) {
    const Share o = shape_of(a, order[k]);
    off += (o.N / o.NM) % NG;
  }
  const int g = s.NM, nu = s.N / g, base = nu / NG, extra = nu % NG;
  const int v = ((gi - off) % NG + NG) % NG;
  s.r0 = g * (v * base + min(v, extra));
  s.R = g * (base + (v < extra ? 1 : 0));
  return s;
}

// Weight rows in a weight slot in LDS keep their HBM format (f32, bf16, int8
// codes or 4-bit codes, q4 rows padded to whole KB); the q8 and q4 block
// scales stay beside the weights and multiply each chunk's dot product.  A
// compute chunk is one lane's load: 16 bytes (4 f32, 8 bf16 or 16 int8
// weights) or, for q4, 8 bytes (16 weights), so a block of 64 lanes spans
// 256, 512 or 1,024 weights.  The GEMV widens q8 and q4 chunks to bf16 pairs
// in registers (exact: |q| <= 128, |c - 8| <= 8).
__host__ __device__ constexpr bool chunk16(int wt) { return wt == W_Q8 || wt == W_Q4; }  // 16 weights per chunk
// Bytes of a weight row of width K as stored in HBM.
__host__ __device__ constexpr int raw_rowb(int wt, int K) {
  return wt == W_F32 ? 4 * K : wt == W_BF16 ? 2 * K : wt == W_Q8 ? K : K / 2;
}
// ... and in a weight slot
__host__ __device__ constexpr int slot_rowb(int wt, int K) { return wt == W_Q4 ? (K / 2 + 1023) & ~1023 : raw_rowb(wt, K); }
// weights of one compute block, and a row's compute blocks
__host__ __device__ constexpr int block_weights(int wt) { return wt == W_F32 ? 256 : wt == W_BF16 ? 512 : 1024; }
__host__ __device__ constexpr int row_blocks(int wt, int K) { return K / block_weights(wt); }
// compute blocks a row of width H may span: its normalized operand lives in
// registers (a 16-weight chunk takes twice the operand words of a bf16 one)
__host__ __device__ constexpr int nb_hidden(int wt) { return chunk16(wt) ? 1 : 2; }
// compute blocks of the O and down rows (widths nq*hd and F), whose operand
// chunks are also held in registers per item
__host__ __device__ constexpr int nb_wide(int wt) { return chunk16(wt) ? 4 : 6; }
// one lane's weight chunk
template <int WT> struct WChunk { typedef uint4 T; };
template <> struct WChunk<W_Q4> { typedef uint2 T; };

// weight row (bytes rb in HBM) and block-scale row of output row n, matrix mat
__device__ __forceinline__ void wrow_of(const FrameArgs &a, const Common &cm, const Ph &p, int n, int mat,
                                        int K, int rb, const uint8_t *&w, const uint8_t *&sc) {
  const int qd = a.nq * a.hd, kd = a.nkv * a.hd;
  int which = 0, r = n;
  if (p.type == PH_HEAD) {
    const int hi = p.stack ? 0 : 1 + p.step;
    w = (const uint8_t *)cm.head_w[hi] + (size_t)n * rb;
    sc = cm.head_sc[hi] ? (const uint8_t *)(cm.head_sc[hi] + (size_t)n * (K / 32)) : nullptr;
    return;
  }
  switch (p.type) {
    case PH_QKV:
      if (n < qd) which = LW_Q;
      else if (n < qd + kd) { which = LW_K; r = n - qd; }
      else { which = LW_V; r = n - qd - kd; }
      break;
    case PH_O: which = LW_O; break;
    case PH_GU: which = mat ? LW_U : LW_G; break;
    default: which = LW_D; break;
  }
  const LayerTab &T = tab_of(a, cm, p.stack, p.layer);
  w = (const uint8_t *)T.w[which] + (size_t)r * rb;
  sc = T.sc[which] ? (const uint8_t *)(T.sc[which] + (size_t)r * (K / 32)) : nullptr;
}
__device__ __forceinline__ const void *gain_of(const FrameArgs &a, const Common &cm, const Ph &p) {
  if (p.type == PH_QKV) return tab_of(a, cm, p.stack, p.layer).attn_norm;
  if (p.type == PH_GU) return tab_of(a, cm, p.stack, p.layer).mlp_norm;
  if (p.type == PH_HEAD) return p.stack ? a.t_norm : a.p_norm;
  return nullptr;
}
// slot layout: weights [R*NM rows] (slot_rowb bytes each), block scales
// [R*NM][K/32] (q8 / q4, 1 KB aligned), gain [H].
template <int WT>
__device__ __forceinline__ uint32_t scales_off(const Share &s) { return (uint32_t)(s.R * s.NM) * slot_rowb(WT, s.K); }
template <int WT>
__device__ __forceinline__ uint32_t gain_off(const Share &s) {
  return scales_off<WT>(s) + (w_blocked(WT) ? up1k((uint32_t)(s.R * s.NM) * (s.K / 16)) : 0u);
}

// Issue this loader wave's part of the direct-to-LDS loads of phase p's
// weight slice: loader wave li takes weight blocks [li nb / NLW, (li + 1) nb /
// NLW) and the last one also the block scales and the norm gain.  Every 1 KB
// block is one instruction.  A wave can keep only a limited number of these
// loads in flight, so several loader waves land a slice sooner.
template <int WT>
__device__ __forceinline__ void dma_slice(const FrameArgs &a, const Common &cm, const Ph &p, uint32_t slot) {
  const int lane = threadIdx.x & 63;
  const int li = (int)(threadIdx.x >> 6) - NW;
  const Share s = cm.sh[p.type];
  // rows of rb bytes in 1 KB blocks, block b at b KB; in a q4 row's last
  // block lanes past its end load its last chunk again (so that every lane
  // of every load is on: a lane mask here slows the whole slice's issue)
  const int rb = raw_rowb(WT, s.K), bpr = (rb + 1023) >> 10, U = s.R * s.NM;
  const int nb = U * bpr, b1 = (li + 1) * nb / NLW;
  for (int b = li * nb / NLW; b < b1;) {
    const int u = b / bpr;
    const uint8_t *w, *sc;
    wrow_of(a, cm, p, s.r0 + u / s.NM, u % s.NM, s.K, rb, w, sc);
    for (int cb = b - u * bpr; cb < bpr && b < b1; ++cb, ++b) {
      if constexpr (WT == W_Q4) dma16(w + min(cb * 1024 + lane * 16, rb - 16), slot + (uint32_t)b * 1024u);
      else dma16(w + cb * 1024 + lane * 16, slot + (uint32_t)b * 1024u);
    }
  }
  if (li != NLW - 1) return;
  if constexpr (w_blocked(WT)) {
    const int spu = s.K / 256, n = U * spu;  // 16-byte scale chunks per row, in all
    const uint32_t so = scales_off<WT>(s);
    for (int sb = 0; sb * 64 < n; ++sb) {
      const int idx = min(sb * 64 + lane, n - 1);
      const int u = idx / spu, k = idx - u * spu;
      const uint8_t *w, *sc;
      wrow_of(a, cm, p, s.r0 + u / s.NM, u % s.NM, s.K, rb, w, sc);
      dma16(sc + k * 16, slot + so + (uint32_t)sb * 1024u);
    }
  }
  const void *g = gain_of(a, cm, p);
  if (g) {
    const int n = a.H * (a.tab_bf16 ? 2 : 4) / 16;
    const uint32_t go = gain_off<WT>(s);
    for (int gb = 0; gb * 64 < n; ++gb)
      dma16((const uint8_t *)g + min(gb * 64 + lane, n - 1) * 16, slot + go + (uint32_t)gb * 1024u);
  }
}

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), c, false);
}
// int8 bytes b, b+1 of w as a bf16 pair (exact: |q| <= 128)
__device__ __forceinline__ uint32_t i8pair(uint32_t w, int b) {
  const float lo = (float)(int8_t)(w >> (8 * b)), hi = (float)(int8_t)(w >> (8 * b + 8));
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}
// The 8 4-bit codes of w (low nibble first) as 4 bf16 pairs c - 8 (exact):
// each code c becomes the f32 2^23 + c by a byte permute (bits 0x4b0000cc),
// 2^23 + 8 is subtracted (exact), and a pair keeps the two results' high
// halves (small integers have no low mantissa bits).
__device__ __forceinline__ void q4pairs8(uint32_t w, uint32_t *p) {
  const uint32_t ev = w & 0x0f0f0f0fu, od = (w >> 4) & 0x0f0f0f0fu;  // codes 0, 2, 4, 6 and 1, 3, 5, 7 as bytes
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t sel = 0x070c0c00u | (uint32_t)k;  // byte k of the second source, 0, 0, 0x4b
    const float lo = __uint_as_float(__builtin_amdgcn_perm(0x4b000000u, ev, sel)) - 8388616.0f;
    const float hi = __uint_as_float(__builtin_amdgcn_perm(0x4b000000u, od, sel)) - 8388616.0f;
    p[k] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
}

// The operand elements that meet one weight chunk in LDS: 8 bf16 pairs for
// q8 and q4 (a, b), 4 pairs for bf16 (a), 4 floats for f32 (a).
struct OpC {
  uint4 a, b;
};
// chunk c of an operand row in LDS
template <int WT>
__device__ __forceinline__ OpC op_lds(const uint32_t *op, int c) {
  OpC x;
  if constexpr (chunk16(WT)) {
    x.a = ((const uint4 *)op)[2 * c];
    x.b = ((const uint4 *)op)[2 * c + 1];
  } else {
    x.a = ((const uint4 *)op)[c];
    x.b = x.a;
  }
  return x;
}

// a weight chunk of a row (in LDS) . its operand elements: a q8 or q4 chunk
// is 16 codes, half a 32-weight scale block, whose scale multiplies the
// chunk's dot product
template <int WT>
__device__ __forceinline__ float chunk_dot(typename WChunk<WT>::T w, const OpC &x, float scale) {
  if constexpr (WT == W_F32) {
    return __uint_as_float(w.x) * __uint_as_float(x.a.x) + __uint_as_float(w.y) * __uint_as_float(x.a.y) +
           __uint_as_float(w.z) * __uint_as_float(x.a.z) + __uint_as_float(w.w) * __uint_as_float(x.a.w);
  } else if constexpr (WT == W_Q8) {
    float s = dot2(i8pair(w.x, 0), x.a.x, 0.f);
    s = dot2(i8pair(w.x, 2), x.a.y, s);
    s = dot2(i8pair(w.y, 0), x.a.z, s);
    s = dot2(i8pair(w.y, 2), x.a.w, s);
    s = dot2(i8pair(w.z, 0), x.b.x, s);
    s = dot2(i8pair(w.z, 2), x.b.y, s);
    s = dot2(i8pair(w.w, 0), x.b.z, s);
    s = dot2(i8pair(w.w, 2), x.b.w, s);
    return s * scale;
  } else if constexpr (WT == W_Q4) {
    uint32_t p[8];
    q4pairs8(w.x, p);
    q4pairs8(w.y, p + 4);
    float s = dot2(p[0], x.a.x, 0.f);
    s = dot2(p[1], x.a.y, s);
    s = dot2(p[2], x.a.z, s);
    s = dot2(p[3], x.a.w, s);
    s = dot2(p[4], x.b.x, s);
    s = dot2(p[5], x.b.y, s);
    s = dot2(p[6], x.b.z, s);
    s = dot2(p[7], x.b.w, s);
    return s * scale;
  } else {
    return dot2(w.w, x.a.w, dot2(w.z, x.a.z, dot2(w.y, x.a.y, dot2(w.x, x.a.x, 0.f))));
  }
}

// Barrier of the compute waves (the loader waves never join it): an arrival
// counter in LDS; gen counts this wave's barriers times NW.
__device__ __forceinline__ bool cbar(const FrameArgs &a, Common &cm, uint32_t &gen) {
  gen += NW;
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(&cm.cbar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  for (uint32_t spins = 0; __hip_atomic_load(&cm.cbar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < gen; ++spins) {
    if (spins > SPIN_LIMIT) {
      err_set(a.err);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// 1 / RMS of a row from the compute waves' partial sums of squares (LDS).
__device__ __forceinline__ float rms_inv(const FrameArgs &a, const float *pss) {
  float ss = pss[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) ss += pss[w];
  // mean by the hardware reciprocal of H (exact for a power of two) and
  // v_rsq_f32 (1 ulp): a handful of instructions on the critical path
  return __builtin_amdgcn_rsqf(ss * __builtin_amdgcn_rcpf((float)a.H) + a.eps);
}
// gain element e of a norm table (bf16 or f32) staged in LDS
__device__ __forceinline__ float gain_at(const FrameArgs &a, const uint8_t *g, int e) {
  return a.tab_bf16 ? __uint_as_float((uint32_t)((const uint16_t *)g)[e] << 16) : ((const float *)g)[e];
}
// bf16 pairs of RMSNorm(x) * g for elements e0 .. e0 + 7
// (bf16, q8 and q4 weights run with bf16 tables and gains, f32 weights with f32
// ones: the kernel's weight type fixes the gains' format at compile time)
template <bool TB>
__device__ __forceinline__ uint4 norm8(const FrameArgs &a, const float *x, const uint8_t *g, float r, int e0) {
  const float4 x0 = *(const float4 *)(x + e0), x1 = *(const float4 *)(x + e0 + 4);
  float g8[8];
  if constexpr (TB) {
    const uint4 gw = *(const uint4 *)(g + 2 * e0);
    g8[0] = lo16(gw.x); g8[1] = hi16(gw.x); g8[2] = lo16(gw.y); g8[3] = hi16(gw.y);
    g8[4] = lo16(gw.z); g8[5] = hi16(gw.z); g8[6] = lo16(gw.w); g8[7] = hi16(gw.w);
  } else {
    const float4 g0 = *(const float4 *)(g + 4 * e0), g1 = *(const float4 *)(g + 4 * e0 + 16);
    g8[0] = g0.x; g8[1] = g0.y; g8[2] = g0.z; g8[3] = g0.w;
    g8[4] = g1.x; g8[5] = g1.y; g8[6] = g1.z; g8[7] = g1.w;
  }
  return make_uint4(pack2(x0.x * r * g8[0], x0.y * r * g8[1]), pack2(x0.z * r * g8[2], x0.w * r * g8[3]),
                    pack2(x1.x * r * g8[4], x1.y * r * g8[5]), pack2(x1.z * r * g8[6], x1.w * r * g8[7]));
}
// The operand elements of weight chunk c for a row of width H: RMSNorm(x) * g,
// rounded as an operand row would be, built in registers from the residual row.
template <int WT>
__device__ __forceinline__ OpC norm_chunk(const FrameArgs &a, const float *x, const uint8_t *g, float r, int c) {
  OpC o;
  if constexpr (chunk16(WT)) {
    o.a = norm8<true>(a, x, g, r, 16 * c);
    o.b = norm8<true>(a, x, g, r, 16 * c + 8);
  } else if constexpr (WT != W_F32) {
    o.a = norm8<true>(a, x, g, r, 8 * c);
    o.b = o.a;
  } else {
    const int e0 = 4 * c;
    const float4 xv = *(const float4 *)(x + e0);
    float y[4] = {xv.x * r * gain_at(a, g, e0), xv.y * r * gain_at(a, g, e0 + 1), xv.z * r * gain_at(a, g, e0 + 2),
                  xv.w * r * gain_at(a, g, e0 + 3)};
    if (a.act_bf16)
      for (int j = 0; j < 4; ++j) y[j] = bf16_rne(y[j]);
    o.a = make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3]));
    o.b = o.a;
  }
  return o;
}

// table row (bf16 or f32) element pairs of this thread -> v[2 * HPAIR]
// (zero beyond the row: every element is written, so no value is carried
// over from an earlier phase)
// (TB: bf16 tables, which every kernel but the f32 one has)
template <bool TB>
__device__ __forceinline__ void tab_pairs(const FrameArgs &a, const void *tab, size_t row, float *v) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < HPAIR; ++k) {
    const int pi = tid + k * NT;
    v[2 * k] = 0.f;
    v[2 * k + 1] = 0.f;
    if (2 * pi < a.H) {
      if constexpr (TB) {
        const uint32_t w = ld((const uint32_t *)((const uint16_t *)tab + row * a.H) + pi);
        v[2 * k] = lo16(w); v[2 * k + 1] = hi16(w);
      } else {
        const uint64_t f = ld((const uint64_t *)((const float *)tab + row * a.H) + pi);
        v[2 * k] = __uint_as_float((uint32_t)f); v[2 * k + 1] = __uint_as_float((uint32_t)(f >> 32));
      }
    }
  }
}

// argmax over the workgroups' partial maxima of the head with tag; lowest
// index wins ties.  Compute waves; false on timeout.
// Logit -> unsigned key in the same order (-0 and +0 equal, as they compare).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x == 0.f ? 0.f : x);
  return b ^ ((b >> 31) ? 0xffffffffu : 0x80000000u);
}

// The sampled code under top-k.  Every compute thread polls its share of the
// head's Vc logits into LDS (logit i = u * NT + tid is value u of the
// thread).  The k-th largest key is found by a radix select, 8 bits per pass
// from the top: every thread adds its keys to an LDS histogram, wave 0 scans
// it, picks the digit and clears it for the next pass.  After the last pass
// wave 0 also finds, among the logits equal to the threshold, the index of
// the last member: equal logits count in index order, lower indices first
// (the argmax's tie rule).  Then every thread scores the members among its
// logits (code j of frame position q) and the best score wins; every other
// logit scores -inf.  Values are read back from LDS at each use: this runs
// inside the phase loop, where registers are scarce.
__device__ __forceinline__ bool resolve_top_k(const FrameArgs &a, Common &cm, uint32_t &gen, uint32_t *scratch,
                                              uint32_t tag, int q, int j) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, Vc = a.Vc;
  if (tid < 256) cm.hist[tid] = 0;
  if (!poll_lin(a, a.lgx, Vc, tag, scratch)) cm.abort = 1;
  if (!cbar(a, cm, gen) || cm.abort) return false;
  auto key_at = [&](int i) { return order_key(__uint_as_float(scratch[min(i, Vc - 1)])); };
  uint32_t prefix = 0, need = (uint32_t)a.top_k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hmask = pass ? 0xffffffffu << (shift + 8) : 0u;
    for (int u = 0; u < TKU; ++u) {
      const uint32_t key = key_at(u * NT + tid);
      if (u * NT + tid < Vc && (key & hmask) == prefix) atomicAdd(&cm.hist[(key >> shift) & 255], 1u);
    }
    if (!cbar(a, cm, gen)) return false;
    if (wave == 0) {
      // lane l holds bins 255 - 4l .. 252 - 4l (descending); inclusive scan over lanes
      uint32_t c[4], c4 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) { c[e] = cm.hist[255 - 4 * lane - e]; c4 += c[e]; }
      uint32_t cum = c4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(cum, o, 64);
        if (lane >= o) cum += t;
      }
      const uint64_t hit = __ballot(cum >= need);
      const int hl = (int)__ffsll((unsigned long long)hit) - 1;  // the lane whose bins reach the k-th
      uint32_t bin = 0, rest = 0, run = cum - c4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (run + c[e] >= need) { bin = (uint32_t)(255 - 4 * lane - e); rest = need - run; break; }
        run += c[e];
      }
      prefix |= (uint32_t)__builtin_amdgcn_readlane((int)bin, hl) << shift;
      need = (uint32_t)__builtin_amdgcn_readlane((int)rest, hl);
#pragma unroll
      for (int e = 0; e < 4; ++e) cm.hist[4 * lane + e] = 0;  // (every lane has read its bins)
      if (pass == 3) {
        // the need-th logit equal to the threshold, in index order: the last member
        int last = -1;
        uint32_t seen = 0;
        for (int i0 = 0; i0 < Vc && last < 0; i0 += 64) {
          const uint64_t eq = __ballot(i0 + lane < Vc && key_at(i0 + lane) == prefix);
          const uint32_t n = (uint32_t)__popcll(eq);
          if (seen + n >= need) {
            uint64_t m = eq;
            for (uint32_t r = seen + 1; r < need; ++r) m &= m - 1;  // drop the lower need - seen - 1
            last = i0 + (int)__ffsll((unsigned long long)m) - 1;
          }
          seen += n;
        }
        need = (uint32_t)last;
      }
      if (lane == 0) { cm.tsel[0] = prefix; cm.tsel[1] = need; }
    }
    if (!cbar(a, cm, gen)) return false;
    prefix = cm.tsel[0];
    need = cm.tsel[1];
  }
  const int last = (int)need;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int u = 0; u < TKU; ++u) {
    const int i = u * NT + tid;
    const uint32_t key = key_at(i);
    if (i < Vc && (key > prefix || (key == prefix && i <= last)))
      pick(bv, bi, sample_score(__uint_as_float(scratch[i]), a.inv_temp, a.seed, 0, q, j, i), i);
  }
  wave_argmax(bv, bi);
  if (lane == 0) { cm.amv[wave] = bv; cm.ami[wave] = bi; }
  if (!cbar(a, cm, gen)) return false;
  float b2 = cm.amv[0];
  int i2 = cm.ami[0];
  for (int w = 1; w < NW; ++w) pick(b2, i2, cm.amv[w], cm.ami[w]);
  cm.code = i2 == 0x7fffffff ? 0 : i2;  // every thread writes the same value
  return true;
}

// The code a head decided: the best of the GEMV workgroups' (value, index)
// words, or under top-k sampling the pick among all the head's logits (q, j:
// the code's frame position and index, its sampling key).
template <bool SMP>
__device__ __forceinline__ bool resolve_code(const FrameArgs &a, Common &cm, uint32_t &gen, uint32_t *scratch,
                                             int NG, uint32_t tag, int q, int j) {
  if constexpr (SMP) {
    if (a.top_k > 0) return resolve_top_k(a, cm, gen, scratch, tag, q, j);
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (!poll_lin(a, a.amax, 2 * NG, tag, scratch)) cm.abort = 1;
  if (!cbar(a, cm, gen) || cm.abort) return false;  // each thread reduces words other threads polled
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int w = tid; w < NG; w += NT) pick(bv, bi, __uint_as_float(scratch[2 * w]), (int)scratch[2 * w + 1]);
  wave_argmax(bv, bi);
  if (lane == 0) { cm.amv[wave] = bv; cm.ami[wave] = bi; }
  if (!cbar(a, cm, gen)) return false;
  float b2 = cm.amv[0];
  int i2 = cm.ami[0];
  for (int w = 1; w < NW; ++w) pick(b2, i2, cm.amv[w], cm.ami[w]);
  cm.code = i2 == 0x7fffffff ? 0 : i2;  // every thread writes the same value
  return true;
}

// One wave's GEMV items of the slice (UPI weight rows each: 1, or the gate and
// up rows of a row pair), round-robin over the compute waves; the results of
// item it go to out(it, acc) as uniform values.  A row is at most MAXB 1 KB
// blocks; an item's weight chunks are all loaded before its dot products.
// op(m, cb, c) gives operand row m's elements for chunk c (block cb);
// pre(it) is read when item it starts and handed to out(it, acc, pre).
struct NoPre {
  __device__ __forceinline__ float operator()(int) const { return 0.f; }
};
// Items go round-robin: this wave takes items wv, wv + nwv, ...
// MC: the operand row count at compile time (1 or 2; 0: the run-time M)
template <int WT, int UPI, int MAXB, int MC, class Op, class Out, class Pre = NoPre>
__device__ __forceinline__ void gemv_items(const uint8_t *slot, Op op, const Share &s, int Mrt, Out out,
                                           Pre pre = Pre(), int wv = -1, int nwv = NW) {
  const int M = MC ? MC : Mrt;
  typedef typename WChunk<WT>::T WCh;
  const int lane = threadIdx.x & 63;
  const int rowb = slot_rowb(WT, s.K), bpr = row_blocks(WT, s.K);
  const int nitems = s.R * s.NM / UPI;
  const uint8_t *scb = slot + scales_off<WT>(s);
  for (int it = wv < 0 ? (int)(threadIdx.x >> 6) : wv; it < nitems; it += nwv) {
    // Every block's loads are unconditional, from block min(cb, bpr - 1)
    // past the row's end (read, never used): a load under a branch makes the
    // compiler wait for all outstanding LDS operations where the branch joins.
    WCh w[UPI][MAXB];
#pragma unroll
    for (int q = 0; q < UPI; ++q)
#pragma unroll
      for (int cb = 0; cb < MAXB; ++cb)
        w[q][cb] = ((const WCh *)(slot + (size_t)(it * UPI + q) * rowb))[min(cb, bpr - 1) * 64 + lane];
    // q8 / q4: each chunk's block scale (chunk c of 16 codes: scale c / 2),
    // requested with the weights
    float scv[UPI][MAXB];
#pragma unroll
    for (int q = 0; q < UPI; ++q)
#pragma unroll
      for (int cb = 0; cb < MAXB; ++cb) {
        if constexpr (w_blocked(WT)) {
          const uint16_t *scl = (const uint16_t *)(scb + (size_t)(it * UPI + q) * (s.K / 16));
          scv[q][cb] = f16_to_f32(scl[(min(cb, bpr - 1) * 64 + lane) >> 1]);
        } else {
          scv[q][cb] = 1.f;
        }
      }
    const float pv = pre(it);
    // the operand chunks too, before any dot product (from LDS they would
    // otherwise wait one LDS round trip per block)
    OpC x[2][MAXB];
#pragma unroll
    for (int cb = 0; cb < MAXB; ++cb) {
      const int c = min(cb, bpr - 1) * 64 + lane;  // (register operands take cb itself)
      x[0][cb] = op(0, cb, c);
      if (M > 1) x[1][cb] = op(1, cb, c);
    }
    float acc[UPI][2];
#pragma unroll
    for (int q = 0; q < UPI; ++q) acc[q][0] = acc[q][1] = 0.f;
#pragma unroll
    for (int cb = 0; cb < MAXB; ++cb) {
      // Every block's products are computed (past the row's end from the
      // clamped block, then dropped by a select): with a branch here the
      // compiler sinks each block's loads behind it, one LDS round trip per
      // block instead of one per item.
      const bool on = cb < bpr;
#pragma unroll
      for (int q = 0; q < UPI; ++q) {
        const float d0 = chunk_dot<WT>(w[q][cb], x[0][cb], scv[q][cb]);
        acc[q][0] += on ? d0 : 0.f;
        if (M > 1) {
          const float d1 = chunk_dot<WT>(w[q][cb], x[1][cb], scv[q][cb]);
          acc[q][1] += on ? d1 : 0.f;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < UPI; ++q) {
      acc[q][0] = wave_sum(acc[q][0]);
      if (M > 1) acc[q][1] = wave_sum(acc[q][1]);
    }
    out(it, acc, pv);
  }
}

// The QKV or gate/up phase's items of one wave (index wv of nwv): the
// normalized operand built in registers from the residual rows, then QKV rows
// (published as they are) or gate/up row pairs (z = SiLU(g) * u published as
// the down projection's operand).  With two weight slots the loader waves take
// items too: these slices' rows do not divide evenly over the compute waves.
template <int WT, int MC>
__device__ __forceinline__ void normed_items_m(const FrameArgs &a, const Common &cm, int type, const float *xres,
                                               const uint8_t *sp, uint32_t tag, int wv, int nwv) {
  constexpr int M = MC;  // operand rows, at compile time
  constexpr int NBH = nb_hidden(WT);
  const int lane = threadIdx.x & 63;
  const Share s = cm.sh[type];
  const uint8_t *gain = sp + gain_off<WT>(s);
  const int bpr = row_blocks(WT, a.H);
  const float r0 = rms_inv(a, cm.pss[0]), r1 = M > 1 ? rms_inv(a, cm.pss[1]) : 0.f;
  OpC xo[2][NBH];
#pragma unroll
  for (int cb = 0; cb < NBH; ++cb) {  // unconditional loads (see gemv_items)
    const int c = min(cb, bpr - 1) * 64 + lane;
    xo[0][cb] = norm_chunk<WT>(a, xres, gain, r0, c);
    if (M > 1) xo[1][cb] = norm_chunk<WT>(a, xres + a.H, gain, r1, c);
  }
  auto op = [&](int m, int cb, int) -> OpC { return xo[m][cb]; };
  if (type == PH_QKV) {
    auto out = [&](int it, float (&acc)[1][2], float) {
      if (lane < M) tputf(a.qkvb + (size_t)lane * s.N + s.r0 + it, lane ? acc[0][1] : acc[0][0], tag);
    };
    if (M > 1) gemv_items<WT, 1, NBH, 2>(sp, op, s, M, out, NoPre(), wv, nwv);
    else gemv_items<WT, 1, NBH, 1>(sp, op, s, M, out, NoPre(), wv, nwv);
    return;
  }
  // item = row pair (2 p, 2 p + 1)
  auto out = [&](int it, float (&acc)[4][2], float) {
    for (int m = 0; m < M; ++m) {
      // SiLU(g) * u with the hardware exp and reciprocal (a few ulp)
      const float z0 = acc[0][m] * __builtin_amdgcn_rcpf(1.0f + __expf(-acc[0][m])) * acc[1][m];
      const float z1 = acc[2][m] * __builtin_amdgcn_rcpf(1.0f + __expf(-acc[2][m])) * acc[3][m];
      if constexpr (WT != W_F32) {  // bf16 operands (every kernel but the f32 one has them)
        if (lane < a.rep) tput(a.zb + lane * a.rep_stride + (size_t)m * (a.F / 2) + s.r0 / 2 + it, pack2(z0, z1), tag);
      } else if (lane < 2 * a.rep) {
        const int e = lane & 1;
        tputf(a.zb + (lane >> 1) * a.rep_stride + (size_t)m * a.F + s.r0 + 2 * it + e, e ? z1 : z0, tag);
      }
    }
  };
  if (M > 1) gemv_items<WT, 4, NBH, 2>(sp, op, s, M, out, NoPre(), wv, nwv);
  else gemv_items<WT, 4, NBH, 1>(sp, op, s, M, out, NoPre(), wv, nwv);
}

// one or two operand rows (two only in the predictor's first step), at compile time
template <int WT>
__device__ __forceinline__ void normed_items(const FrameArgs &a, const Common &cm, int type, const float *xres,
                                             const uint8_t *sp, int M, uint32_t tag, int wv, int nwv) {
  if (M > 1) normed_items_m<WT, 2>(a, cm, type, xres, sp, tag, wv, nwv);
  else normed_items_m<WT, 1>(a, cm, type, xres, sp, tag, wv, nwv);
}

// The loader waves: stream each GEMV phase's weight slice (a part each) into
// its LDS slot one phase ahead and meet the compute waves once per phase,
// right after their inputs are in.
template <int WT, bool TRC>
__device__ __forceinline__ void loader_role(const FrameArgs &a, Common &cm, const Lds &L, unsigned char *smem) {
  uint8_t *const p0 = smem + L.slot0, *const p1 = smem + L.slot1;
  Ph cur{PH_QKV, 0, 0, 0, 0};
  dma_slice<WT>(a, cm, cur, lds_addr(p0));
  wait_vm();
  if (TRC && a.trace) cm.ltime = wall_clock64();
  int slot = 0;
  uint32_t done = 0;          // GEMV completions expected so far
  uint32_t seq = 1;           // phase index of cur + 1 (its tag is tag_base + seq)
  bool have_next = false;     // the next phase's slice was issued during the last phase
  // until every wave has finished the current phase's GEMV items
  auto wait_gemv = [&]() -> bool {
    for (uint32_t spins = 0; __hip_atomic_load(&cm.gdone, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < done;
         ++spins) {
      if (spins > SPIN_LIMIT) { err_set(a.err); return false; }
      __builtin_amdgcn_s_sleep(2);
    }
    return true;
  };
  while (cur.type != PH_END) {
    const Ph ng = next_gemv_phase(a, cur, a.pos0);
    __syncthreads();  // the compute waves have this phase's inputs (and are done with the last phase's slot)
    if (cm.abort) break;
    uint8_t *const cslot = slot ? p1 : p0, *const nslot = a.two_slots && !slot ? p1 : p0;
    const bool items = a.two_slots && (cur.type == PH_GU || cur.type == PH_QKV);
    done += items ? NW + NLW : NW;  // this phase's GEMV completions (the loader waves' items too)
    if (items) {
      // its items first (the next phase waits for every one of them), then
      // the next slice; the count tells every loader wave when this slot's
      // rows are no longer read
      const int M = cur.stack == 0 && cur.step == 0 ? 2 : 1;
      normed_items<WT>(a, cm, cur.type, (const float *)(smem + L.xres), cslot, M, a.tag_base + seq,
                       (int)(threadIdx.x >> 6), NW + NLW);
      if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(&cm.gdone, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (ng.type != PH_END && !have_next) {
      if (!a.two_slots && !wait_gemv()) break;  // one slot: it is free once this phase's GEMV is done
      dma_slice<WT>(a, cm, ng, lds_addr(nslot));
    }
    have_next = false;
    if (a.two_slots && cur.type == PH_QKV && ng.type == PH_O) {
      // The attention window: the compute waves only poll until attention is
      // done, so the gate/up slice (the largest) streams into this phase's
      // slot as soon as every GEMV of this phase is done (the loader waves'
      // items included), instead of competing later with the exchange before
      // the gate/up phase.
      const Ph n2 = next_gemv_phase(a, ng, a.pos0);
      if (!wait_gemv()) break;
      dma_slice<WT>(a, cm, n2, lds_addr(cslot));
      have_next = true;  // not loaded again at the O phase's meeting
    }
    wait_vm();
    if (TRC && a.trace) cm.ltime = wall_clock64();
    if (a.two_slots) slot ^= 1;
    for (Ph q = next_phase(a, cur, a.pos0); ; q = next_phase(a, q, a.pos0)) {  // the phase index of ng
      ++seq;
      if (q.type != PH_ATTN && q.type != PH_COMB) break;
    }
    cur = ng;
  }
  wait_vm();  // no load left in flight at exit (after an abort)
}

// SMP: the heads' codes are sampled (sampler.h), else greedy; a compile-time
// switch, so the greedy kernel carries no sampling code.  TRC: the kernel
// stamps its phases (QT_F_TRACE); the other kernels carry no stamp code.
template <int WT, bool SMP, bool TRC>
__device__ __forceinline__ void gemv_role(const FrameArgs &a, unsigned char *smem) {
  Common &cm = *reinterpret_cast<Common *>(smem);
  const Lds L = lds_layout(a);
  if (threadIdx.x >= NT) {
    // The loader waves issue ahead of the compute wave that shares their
    // SIMD: a weight slice's loads then leave as soon as they are issuable
    // instead of waiting behind the compute waves' polls and dot products.
    __builtin_amdgcn_s_setprio(1);
    loader_role<WT, TRC>(a, cm, L, smem);
    return;
  }
  float *xres = (float *)(smem + L.xres);   // [2][H] residual rows
  uint32_t *opnd = (uint32_t *)(smem + L.opnd);
  const int kop = imax(a.H, imax(a.nq * a.hd, a.F));
  const int opw = imax(imax(a.act_bf16 ? kop / 2 : kop, 2 * a.nwg), (a.Vc + 1) / 2);  // words per operand row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gi = (int)blockIdx.x - a.n_attn, NG = a.nwg - a.n_attn;
  const int H = a.H, G = a.G;
  const int force = ld(a.ctl + 1);
  const int pos0 = a.pos0;
  int c0 = ld(a.c0);
  const bool lead = gi == 0;  // writes state, codes and dumps
  const size_t rsel = (size_t)(blockIdx.x % a.rep) * a.rep_stride;  // the exchange copy this workgroup reads
  const uint64_t *xq = a.xq + rsel;
  uint32_t gen = 0;           // compute-wave barrier count

  // Row state kept across phases, each thread its own element pairs (so no
  // barrier guards them): the bridge row and the frame's running sum of code
  // embedding rows.  They live in LDS, not registers, so that the phase loop
  // carries no register arrays.
  float *brg = (float *)(smem + L.brg), *tacc = (float *)(smem + L.tacc);
#pragma unroll
  for (int k = 0; k < HPAIR; ++k) {
    const int pi = tid + k * NT;
    if (2 * pi < H) {
      const uint64_t b = ld((const uint64_t *)a.bridge + pi);
      brg[2 * pi] = __uint_as_float((uint32_t)b);
      brg[2 * pi + 1] = __uint_as_float((uint32_t)(b >> 32));
    }
  }
  // Loop-carried values must not enter the phase loop with loads in flight:
  // the compiler would then wait for every outstanding memory operation
  // (the last phase's stores included) at each of their copies in the loop.
  wait_vm();

  Ph cur{PH_QKV, 0, 0, 0, 0};
  uint32_t seq = 1;
  int slot = 0;
  bool pending = false;  // the previous GEMV phase was a head
  int pending_idx = 0;   // the code index it decides (0: next frame's code 0)
  int pending_q = 0;     // and that code's frame position (its sampling key, with the index)
  int ntr = 0;

  while (cur.type != PH_END) {
    const Ph nxt = next_phase(a, cur, pos0);
    if (cur.type == PH_ATTN || cur.type == PH_COMB) { ++seq; cur = nxt; continue; }
    const bool tracing = TRC && a.trace && lead && cur.frame == 0 && ntr < 767;
    const uint64_t t0 = tracing ? wall_clock64() : 0;
    const uint32_t tag = a.tag_base + seq, tagp = tag - 1;
    const int f = cur.frame;
    const int pos = pos0 + f;
    const int M = (cur.stack == 0 && cur.step == 0 && cur.type != PH_HEAD) ? 2 : 1;
    const Share s = cm.sh[cur.type];
    const bool normed = cur.type == PH_QKV || cur.type == PH_GU || cur.type == PH_HEAD;
    float ss0 = 0.f, ss1 = 0.f;  // this thread's squares of residual rows 0 and 1
    // Sampling: the Gumbel noise of the head's rows does not depend on the
    // logits, so each lane draws it for one of its wave's items (items
    // wave, wave + NW, ...) before the inputs arrive, while the exchange is
    // in flight; the head phase reads it back by lane.  A talker head decides
    // the next frame's code 0, predictor head j code j + 1 of this frame.
    float gnoise = 0.f;
    if constexpr (SMP) {
      if (cur.type == PH_HEAD) {
        const int item = wave + lane * NW;
        gnoise = gumbel_noise(a.seed, 0, cur.stack ? pos + 1 : pos, cur.stack ? 0 : cur.step + 1,
                              s.r0 + (item < s.R ? item : s.R - 1));
      }
    }
    // every compute wave is done with the last phase's operand and residual rows
    if (!cbar(a, cm, gen)) return;

    // ---- inputs -> xres (residual rows) or opnd (operand rows)
    bool ok = true;
    if (cur.type == PH_QKV && cur.layer == 0) {
      if (pending) {
        if (!resolve_code<SMP>(a, cm, gen, opnd, NG, tagp, pending_q, pending_idx)) { cm.abort = 1; ok = false; }
        else {
          const int c = cm.code;
          if (pending_idx == 0) c0 = c;
          else {
            int32_t *ci = a.cin + (size_t)f * G + pending_idx;
            if (lead && tid == 0) {
              st(a.cout + (size_t)f * G + pending_idx, c);
              if (!force) st(ci, c);
            }
            cm.codes[pending_idx] = force ? ld(ci) : c;  // same value from every thread
          }
        }
        pending = false;
      }
      if (ok) {
        float row[2 * HPAIR];
        if (cur.stack == 0 && cur.step == 0) {
          // frame start: code 0 of the frame, rows [bridge, E_0[code 0]]
          int32_t *ci = a.cin + (size_t)f * G;
          if (lead && tid == 0) {
            st(a.cout + (size_t)f * G, c0);
            if (!force) st(ci, c0);
          }
          const int code0 = force ? ld(ci) : c0;
          cm.codes[0] = code0;
          tab_pairs<WT != W_F32>(a, a.code_emb, (size_t)code0, row);
#pragma unroll
          for (int k = 0; k < HPAIR; ++k) {
            const int pi = tid + k * NT;
            if (2 * pi < H) {
              const float b0 = brg[2 * pi], b1 = brg[2 * pi + 1];
              xres[2 * pi] = b0; xres[2 * pi + 1] = b1;
              xres[H + 2 * pi] = row[2 * k]; xres[H + 2 * pi + 1] = row[2 * k + 1];
              ss0 += b0 * b0 + b1 * b1;
              ss1 += row[2 * k] * row[2 * k] + row[2 * k + 1] * row[2 * k + 1];
              tacc[2 * pi] = 0.f + row[2 * k];
              tacc[2 * pi + 1] = 0.f + row[2 * k + 1];
            }
          }
        } else if (cur.stack == 0) {
          tab_pairs<WT != W_F32>(a, a.code_emb, (size_t)cur.step * a.Vc + cm.codes[cur.step], row);
#pragma unroll
          for (int k = 0; k < HPAIR; ++k) {
            const int pi = tid + k * NT;
            if (2 * pi < H) {
              xres[2 * pi] = row[2 * k]; xres[2 * pi + 1] = row[2 * k + 1];
              ss0 += row[2 * k] * row[2 * k] + row[2 * k + 1] * row[2 * k + 1];
              tacc[2 * pi] += row[2 * k];
              tacc[2 * pi + 1] += row[2 * k + 1];
            }
          }
        } else {
          // talker input: the frame's G code rows, then the overlay row, in order
          float trow[2 * HPAIR];
          tab_pairs<WT != W_F32>(a, a.code_emb, (size_t)(G - 1) * a.Vc + cm.codes[G - 1], row);
          tab_pairs<WT != W_F32>(a, a.text_emb, (size_t)ld(a.overlay + f), trow);
#pragma unroll
          for (int k = 0; k < HPAIR; ++k) {
            const int pi = tid + k * NT;
            if (2 * pi < H) {
              const float v0 = (tacc[2 * pi] + row[2 * k]) + trow[2 * k];
              const float v1 = (tacc[2 * pi + 1] + row[2 * k + 1]) + trow[2 * k + 1];
              xres[2 * pi] = v0; xres[2 * pi + 1] = v1;
              ss0 += v0 * v0 + v1 * v1;
              if (a.dump && lead) { st(a.x0_dump + 2 * pi, v0); st(a.x0_dump + 2 * pi + 1, v1); }
            }
          }
          if (a.dump && lead && tid <= G) st(a.gather_dump + tid, tid < G ? cm.codes[tid] : ld(a.overlay + f));
          if (a.dump && lead && tid == 0) st(a.tpos_dump, pos);
        }
      }
      // The table loads above are all consumed; saying so here keeps the
      // compiler from waiting on every memory operation (the last phase's
      // stores included) at the top of each later phase.
      wait_vm();
    } else {
      // residual rows (normed phases) or operand rows (O: attention output, D: SiLU-mul output)
      const uint64_t *src = xq;
      int rows = M, w = H, dw = H;
      uint32_t *dst = (uint32_t *)xres;
      if (cur.type == PH_HEAD) {
        if (cur.stack == 0 && cur.step == 0) src += H;  // the code row of the pair
      } else if (cur.type == PH_O || cur.type == PH_D) {
        src = (cur.type == PH_O ? a.ob : a.zb) + rsel;
        const int k = cur.type == PH_O ? a.nq * a.hd : a.F;
        w = a.act_bf16 ? k / 2 : k;
        dst = opnd;
        dw = opw;
      }
      ok = poll_rows(a, src, rows, w, tagp, dst, dw, [&](int i, uint32_t v) {
        const float x = __uint_as_float(v);  // squares feed the RMSNorm of the residual rows
        if (i < w) ss0 += x * x;
        else ss1 += x * x;
      });
    }
    const uint64_t tp = tracing ? wall_clock64() : 0;
    if (!ok) cm.abort = 1;
    if (normed) {
      ss0 = wave_sum(ss0);
      if (M > 1) ss1 = wave_sum(ss1);
      if (lane == 0) { cm.pss[0][wave] = ss0; cm.pss[1][wave] = ss1; }
    }
    __syncthreads();  // with the loader waves: inputs in LDS, this phase's slice landed
    if (cm.abort) return;
    const uint64_t t1 = tracing ? wall_clock64() : 0;
    const uint64_t tl = tracing ? cm.ltime : 0;

    // ---- prologue: the normalized operand rows, each lane its own chunks
    const uint8_t *sp = smem + (slot ? L.slot1 : L.slot0);
    constexpr int NBH = nb_hidden(WT);
    OpC xo[2][NBH];  // [row][block]
    if (normed && !(cur.type == PH_GU || (cur.type == PH_QKV && a.two_slots))) {  // (else inside normed_items)
      const uint8_t *gain = sp + gain_off<WT>(s);
      const int bpr = row_blocks(WT, H);
      const float r0 = rms_inv(a, cm.pss[0]), r1 = M > 1 ? rms_inv(a, cm.pss[1]) : 0.f;
#pragma unroll
      for (int cb = 0; cb < NBH; ++cb) {  // unconditional loads (see gemv_items)
        const int c = min(cb, bpr - 1) * 64 + lane;
        xo[0][cb] = norm_chunk<WT>(a, xres, gain, r0, c);
        if (M > 1) xo[1][cb] = norm_chunk<WT>(a, xres + H, gain, r1, c);
      }
      if (cur.type == PH_HEAD && cur.stack == 1) {
        // the talker's normed output row, kept (unrounded) as the next frame's bridge
#pragma unroll
        for (int k = 0; k < HPAIR; ++k) {
          const int pi = tid + k * NT;
          if (2 * pi < H) {
            const float b0 = xres[2 * pi] * r0 * gain_at(a, gain, 2 * pi);
            const float b1 = xres[2 * pi + 1] * r0 * gain_at(a, gain, 2 * pi + 1);
            brg[2 * pi] = b0;
            brg[2 * pi + 1] = b1;
            if (lead) { st(a.bridge + 2 * pi, b0); st(a.bridge + 2 * pi + 1, b1); }
          }
        }
      }
    }
    auto op_reg = [&](int m, int cb, int) -> OpC { return xo[m][cb]; };
    auto op_row = [&](int m, int, int c) -> OpC { return op_lds<WT>(opnd + m * opw, c); };
    const uint64_t t2 = tracing ? wall_clock64() : 0;

    // ---- GEMV; each wave publishes the rows it computed
    if (cur.type == PH_GU || (cur.type == PH_QKV && a.two_slots)) {
      normed_items<WT>(a, cm, cur.type, xres, sp, M, tag, wave, a.two_slots ? NW + NLW : NW);
    } else if (cur.type == PH_HEAD) {
      // logits and the wave's running argmax, then the workgroup's
      float *lg = cur.stack ? a.logits_t : a.logits_p + (size_t)cur.step * a.Vc;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      gemv_items<WT, 1, NBH, 1>(sp, op_reg, s, 1, [&](int it, float (&acc)[1][2], float) {
        const int n = s.r0 + it;
        if (lane == 0) st(lg + n, acc[0][0]);
        if constexpr (SMP) {
          if (a.top_k > 0 && lane == 0) tputf(a.lgx + n, acc[0][0], tag);  // every logit, for the top-k pick
          // item it is this wave's ((it - wave) / NW)-th: its noise sits in that lane
          const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gnoise), (it - wave) / NW));
          pick(bv, bi, __fadd_rn(__fmul_rn(acc[0][0], a.inv_temp), g), n);
        } else {
          pick(bv, bi, acc[0][0], n);
        }
      });
      if (lane == 0) { cm.amv[wave] = bv; cm.ami[wave] = bi; }
      if (!cbar(a, cm, gen)) return;
      if (tid == 0) {
        for (int w = 1; w < NW; ++w) pick(bv, bi, cm.amv[w], cm.ami[w]);
        tputf(a.amax + 2 * gi, bv, tag);
        tput(a.amax + 2 * gi + 1, (uint32_t)bi, tag);
      }
      pending = true;
      pending_idx = cur.stack ? 0 : cur.step + 1;
      pending_q = cur.stack ? pos + 1 : pos;
    } else {
      const int type = cur.type, N = s.N;
      const bool hid = type == PH_D && cur.stack == 1 && a.dump;
      if (type == PH_QKV) {
        auto out = [&](int it, float (&acc)[1][2], float) {
          if (lane < M) tputf(a.qkvb + (size_t)lane * N + s.r0 + it, lane ? acc[0][1] : acc[0][0], tag);
        };
        if (M > 1) gemv_items<WT, 1, NBH, 2>(sp, op_reg, s, M, out);
        else gemv_items<WT, 1, NBH, 1>(sp, op_reg, s, M, out);
      } else {
        // the residual element (lane: copy lane / M of row lane % M) is read
        // when the item starts, off the path after the reduction
        const int rm = M > 1 ? lane & 1 : 0, rr = M > 1 ? lane >> 1 : lane;
        auto out = [&](int it, float (&acc)[1][2], float res) {
          const int n = s.r0 + it;
          if (lane < M * a.rep) {
            const int m = rm, r = rr;
            const float x = res + (m ? acc[0][1] : acc[0][0]);
            tputf(a.xq + r * a.rep_stride + (size_t)m * H + n, x, tag);
            if (hid && r == 0) st(a.hidden_dump + (size_t)cur.layer * H + n, x);
          }
        };
        auto pre = [&](int it) {  // every lane loads (in bounds), the publishing lanes use it
          const float v = xres[rm * H + s.r0 + it];
          return lane < M * a.rep ? v : 0.f;
        };
        if (M > 1) gemv_items<WT, 1, nb_wide(WT), 2>(sp, op_row, s, M, out, pre);
        else gemv_items<WT, 1, nb_wide(WT), 1>(sp, op_row, s, M, out, pre);
      }
    }
    if (lane == 0)  // this wave is done with the phase's slot
      __hip_atomic_fetch_add(&cm.gdone, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint64_t t3 = tracing ? wall_clock64() : 0;
    if (tracing && tid == 0) {
      uint64_t *tr = a.trace + 8 * ntr;
      st(tr, (uint64_t)cur.type | ((uint64_t)cur.stack << 8) | ((uint64_t)cur.layer << 16) |
                 ((uint64_t)(cur.step & 0xff) << 24));
      st(tr + 1, t0);
      st(tr + 2, t1);
      st(tr + 3, (uint64_t)wall_clock64());
      st(tr + 4, t2);
      st(tr + 5, t3);
      st(tr + 6, tp);  // this wave's inputs were in
      st(tr + 7, tl);  // the phase's weight slice had landed
    }
    if (tracing) ++ntr;
    if (a.two_slots) slot ^= 1;
    ++seq;
    cur = nxt;
  }
  if (TRC && a.trace && lead && tid == 0) st(a.trace + 8 * ntr, (uint64_t)255);
  // the code picked by the last talker head becomes the slot's pending code 0
  if (lead) {
    if (pending) {
      if (!cbar(a, cm, gen) || !resolve_code<SMP>(a, cm, gen, opnd, NG, a.tag_base + seq - 1, pending_q, pending_idx))
        return;
      if (tid == 0) st(a.c0, cm.code);
    }
    if (tid == 0) st(a.pos, pos0 + a.n_frames);
  }
}

// ------------------------------------------------------------ attention role

// An attention event of workgroup (kh, t): predictor (frame, step, layer) or
// talker (frame, layer).
struct Ev {
  int valid, stack, frame, step, layer;
};
__device__ __forceinline__ Ev first_event(const FrameArgs &a, int t, int pos0) {
  if (t == 0) return Ev{1, 0, 0, 0, 0};
  const int f = imax(0, t * TILE - pos0);
  return Ev{f < a.n_frames, 1, f, 0, 0};
}
__device__ __forceinline__ Ev next_event(const FrameArgs &a, Ev e, int t) {
  if (e.stack == 0) {
    if (e.layer + 1 < a.Lp) { ++e.layer; return e; }
    if (e.step + 1 < a.G - 1) { ++e.step; e.layer = 0; return e; }
    e.stack = 1; e.layer = 0; e.step = 0;
    return e;
  }
  if (e.layer + 1 < a.Lt) { ++e.layer; return e; }
  e.frame += 1;
  e.layer = 0;
  e.valid = e.frame < a.n_frames;
  if (t == 0) e.stack = 0;
  return e;
}

template <bool KVB> struct KvT;
template <> struct KvT<true> { static constexpr int esz = 2; };
template <> struct KvT<false> { static constexpr int esz = 4; };

// K/V chunk (16 bytes) -> floats
template <bool KVB>
__device__ __forceinline__ void unpack16(uint4 w, float *v) {
  if constexpr (KVB) {
    v[0] = lo16(w.x); v[1] = hi16(w.x); v[2] = lo16(w.y); v[3] = hi16(w.y);
    v[4] = lo16(w.z); v[5] = hi16(w.z); v[6] = lo16(w.w); v[7] = hi16(w.w);
  } else {
    v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
  }
}

template <int HD, int GQ, bool KVB, bool TRC>
__device__ __forceinline__ void attn_role(const FrameArgs &a, unsigned char *smem) {
  constexpr int ESZ = KvT<KVB>::esz;
  constexpr int ROWB = HD * ESZ;           // bytes per K/V row
  constexpr int DPC = 16 / ESZ;            // dims per 16-byte chunk
  constexpr int CPR = HD / DPC;            // chunks per row (lanes per position)
  constexpr int PG = ANT / CPR;             // position groups
  constexpr int W = (GQ + 2) * HD;         // q | k | v words of one row
  constexpr int NS = ANW / GQ;              // position subsets of P.V
  static_assert(CPR == 16, "K/V rows of 256 bytes");
  static_assert(ANW % GQ == 0 && 2 * 64 >= HD, "P.V wave layout");
  Common &cm = *reinterpret_cast<Common *>(smem);
  const Lds L = lds_layout(a);
  float *rowbuf = (float *)(smem + L.rowbuf);  // [2][GQ + 2][HD]
  float *gq = (float *)(smem + L.gq), *gk = (float *)(smem + L.gk);
  float *rc = (float *)(smem + L.rc), *rs = (float *)(smem + L.rs);  // [2][HD/2]
  float *sc = (float *)(smem + L.sc);          // [GQ][tile]
  float *stat = (float *)(smem + L.stat);      // [GQ][2] max, sum
  float *pvred = (float *)(smem + L.pvred);    // [ANW][GQ][HD]
  uint8_t *kv = smem + L.kv;
  const uint32_t kv_lds = lds_addr(kv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wg = blockIdx.x;
  const int kh = wg % a.nkv, t = wg / a.nkv, ts = t * TILE;
  const int qd = a.nq * HD, kd = a.nkv * HD, nqkv = qd + 2 * kd;
  const int pos0 = a.pos0;
  const int maxT = a.max_tiles;
  const int pg = tid / CPR, cc = tid % CPR;

  // load gains and RoPE rows for event e, then (talker) its K/V tile
  auto prep = [&](const Ev &e) {
    const LayerTab &T = tab_of(a, cm, e.stack, e.layer);
    for (int i = tid; i < HD; i += ANT) {
      gq[i] = a.tab_bf16 ? lo16((uint32_t)ld((const uint16_t *)T.q_norm + i)) : ld((const float *)T.q_norm + i);
      gk[i] = a.tab_bf16 ? lo16((uint32_t)ld((const uint16_t *)T.k_norm + i)) : ld((const float *)T.k_norm + i);
    }
    const int p0 = e.stack ? pos0 + e.frame : (e.step == 0 ? 0 : e.step + 1);
    for (int i = tid; i < HD; i += ANT) {
      const int m = i / (HD / 2), d = i % (HD / 2);
      const int pm = m ? 1 : p0;
      rc[i] = ld(a.rope_cos + (size_t)pm * (HD / 2) + d);
      rs[i] = ld(a.rope_sin + (size_t)pm * (HD / 2) + d);
    }
    wait_vm();
    __syncthreads();
    if (e.stack == 1) {
      // rows [ts, min(p, ts + tile)) of the layer's K and V for this head
      const int p = pos0 + e.frame;
      const int nv = min(p, ts + TILE) - ts;
      if (nv > 0) {
        const size_t hoff = (size_t)e.layer * a.t_layer_stride + (size_t)kh * a.P * HD + (size_t)ts * HD;
        const uint8_t *srcK = a.ring_t + hoff * ESZ;
        const uint8_t *srcV = a.ring_t + (hoff + a.t_kv_stride) * ESZ;
        const int n = nv * ROWB / 16;  // chunks per matrix
        for (int b = wave; b * 64 < n; b += ANW) {
          const int idx = min(b * 64 + lane, n - 1);
          dma16_coherent(srcK + (size_t)idx * 16, kv_lds + (uint32_t)b * 1024u);
          dma16_coherent(srcV + (size_t)idx * 16, kv_lds + (uint32_t)(TILE * ROWB) + (uint32_t)b * 1024u);
        }
      }
    }
  };

  Ev ev = first_event(a, t, pos0);
  if (ev.valid) prep(ev);
  Ph cur{PH_QKV, 0, 0, 0, 0};
  uint32_t seq = 1;
  int ntr = 0;
  while (cur.type != PH_END) {
    const Ph nxt = next_phase(a, cur, pos0);
    const uint32_t tag = a.tag_base + seq, tagp = tag - 1;
    const bool mine = ev.valid && cur.type == PH_ATTN && cur.stack == ev.stack && cur.frame == ev.frame &&
                      cur.layer == ev.layer && (cur.stack == 1 || cur.step == ev.step);
    if (mine) {
      const bool tracing = TRC && a.trace && wg == 0 && cur.frame == 0 && ntr < 255;
      const uint64_t t0 = tracing ? wall_clock64() : 0;
      const int p = pos0 + cur.frame;
      const int M = (cur.stack == 0 && cur.step == 0) ? 2 : 1;
      const int ntile = cur.stack ? ntiles_at(p) : 1;
      // ---- q | k | v rows of this KV head
      uint32_t *rb = (uint32_t *)rowbuf;
      const bool ok = poll<ANT>(a, M * W, tagp, [=](int i) { return rb + i; }, [=](int i) {
        const int m = i / W, r = i - m * W;
        const int off = r < GQ * HD ? kh * GQ * HD + r
                        : r < (GQ + 1) * HD ? qd + kh * HD + (r - GQ * HD)
                                            : qd + kd + kh * HD + (r - (GQ + 1) * HD);
        return a.qkvb + (size_t)m * nqkv + off;
      });
      if (!ok) cm.abort = 1;
      wait_vm();  // the tile's loads (long landed: the poll waited in order)
      __syncthreads();
      if (cm.abort) return;
      const uint64_t t1 = tracing ? wall_clock64() : 0;
      // ---- q/k RMSNorm + RoPE (NeoX halves): one wave per (row, head)
      for (int it = wave; it < M * (GQ + 1); it += ANW) {
        const int m = it / (GQ + 1), h = it % (GQ + 1);
        float *v = rowbuf + (size_t)m * W + h * HD;
        const float *g = h < GQ ? gq : gk;
        const bool act = lane < HD / 2;
        const float x0 = act ? v[lane] : 0.f, x1 = act ? v[lane + HD / 2] : 0.f;
        const float ssum = wave_sum(x0 * x0 + x1 * x1);
        const float r = __builtin_amdgcn_rsqf(ssum / (float)HD + a.eps);
        if (act) {
          const float y0 = x0 * r * g[lane], y1 = x1 * r * g[lane + HD / 2];
          const float c = rc[m * (HD / 2) + lane], sn = rs[m * (HD / 2) + lane];
          v[lane] = y0 * c - y1 * sn;
          v[lane + HD / 2] = y1 * c + y0 * sn;
        }
      }
      __syncthreads();
      // ---- the new K/V rows (set_rows) into LDS and the ring
      uint8_t *kbase, *vbase;
      int base;  // position of LDS row 0
      if (cur.stack) {
        kbase = kv; vbase = kv + TILE * ROWB; base = ts;
      } else {
        kbase = kv + (size_t)cur.layer * 2 * a.Q * ROWB; vbase = kbase + (size_t)a.Q * ROWB; base = 0;
      }
      const bool owner = cur.stack == 0 || p < ts + TILE;
      if (owner) {
        for (int i = tid; i < M * 2 * (ROWB / 8); i += ANT) {
          const int m = i / (2 * (ROWB / 8)), r = i % (2 * (ROWB / 8));
          const int isv = r >= ROWB / 8, wi = r % (ROWB / 8);
          const int pm = cur.stack ? p : (cur.step == 0 ? m : cur.step + 1);
          const float *src = rowbuf + (size_t)m * W + (GQ + isv) * HD + wi * (8 / ESZ);
          uint64_t word;
          if constexpr (KVB)
            word = (uint64_t)pack2(src[0], src[1]) | ((uint64_t)pack2(src[2], src[3]) << 32);
          else
            word = (uint64_t)__float_as_uint(src[0]) | ((uint64_t)__float_as_uint(src[1]) << 32);
          *(uint64_t *)((isv ? vbase : kbase) + (size_t)(pm - base) * ROWB + wi * 8) = word;
          uint8_t *ring;
          if (cur.stack)
            ring = a.ring_t + ((size_t)cur.layer * a.t_layer_stride + (size_t)isv * a.t_kv_stride +
                               (size_t)kh * a.P * HD + (size_t)pm * HD) * ESZ;
          else
            ring = a.ring_p + ((size_t)cur.layer * a.p_layer_stride + (size_t)isv * a.p_kv_stride +
                               (size_t)kh * a.Q * HD + (size_t)pm * HD) * ESZ;
          ring_put(ring + wi * 8, word);
        }
      }
      __syncthreads();
      for (int m = 0; m < M; ++m) {
        const int pm = cur.stack ? p : (cur.step == 0 ? m : cur.step + 1);
        const int n = min(pm - base + 1, cur.stack ? TILE : a.Q);  // valid rows of this tile
        const float *qrow = rowbuf + (size_t)m * W;
        // scores: lanes (pg, chunk cc); 16-lane reduction per position
        float qr[GQ][DPC];
#pragma unroll
        for (int g = 0; g < GQ; ++g)
#pragma unroll
          for (int e = 0; e < DPC; ++e) qr[g][e] = qrow[g * HD + cc * DPC + e];
        for (int j0 = 0; j0 < n; j0 += PG) {
          const int j = j0 + pg;
          float kf[DPC];
          unpack16<KVB>(j < n ? *(const uint4 *)(kbase + (size_t)j * ROWB + cc * 16) : make_uint4(0, 0, 0, 0), kf);
#pragma unroll
          for (int g = 0; g < GQ; ++g) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < DPC; ++e) d += qr[g][e] * kf[e];
            d = row16_sum(d);  // the 16 lanes of a position form one DPP row
            if (cc == 0 && j < n) sc[g * TILE + j] = d * a.scale;
          }
        }
        __syncthreads();
        // softmax statistics: one wave per head
        if (wave < GQ) {
          float mx = -INFINITY;
          for (int j = lane; j < n; j += 64) mx = fmaxf(mx, sc[wave * TILE + j]);
          mx = wave_max(mx);
          float sum = 0.f;
          for (int j = lane; j < n; j += 64) {
            const float e = __expf(sc[wave * TILE + j] - mx);
            sc[wave * TILE + j] = e;
            sum += e;
          }
          sum = wave_sum(sum);
          if (lane == 0) { stat[wave * 2] = mx; stat[wave * 2 + 1] = sum; }
        }
        __syncthreads();
        // P.V: wave w takes query head w % GQ and the positions j = w / GQ
        // (mod NS); each lane two adjacent dims, so no cross-lane reduction
        {
          const int g = wave % GQ, sub = wave / GQ;
          if (2 * lane < HD) {
            float o0 = 0.f, o1 = 0.f;
#pragma unroll 4
            for (int j = sub; j < n; j += NS) {
              const float pj = sc[g * TILE + j];
              float v0, v1;
              if constexpr (KVB) {
                const uint32_t w2 = *(const uint32_t *)(vbase + (size_t)j * ROWB + 4 * lane);
                v0 = lo16(w2); v1 = hi16(w2);
              } else {
                const float2 f2 = *(const float2 *)(vbase + (size_t)j * ROWB + 8 * lane);
                v0 = f2.x; v1 = f2.y;
              }
              o0 += pj * v0;
              o1 += pj * v1;
            }
            *(float2 *)(pvred + (sub * GQ + g) * HD + 2 * lane) = make_float2(o0, o1);
          }
        }
        __syncthreads();
        // sum of the position subsets' partials, element k of [GQ][HD]
        auto pv = [&](int k) {
          float v = 0.f;
#pragma unroll
          for (int w = 0; w < NS; ++w) v += pvred[w * GQ * HD + k];
          return v;
        };
        // publish: normalised output (one tile) or the tile's partial
        if (ntile == 1) {
          // every (word, copy) pair once, spread over the threads
          if (a.act_bf16) {
            for (int i = tid; i < GQ * HD / 2 * a.rep; i += ANT) {
              const int wi = i % (GQ * HD / 2), r = i / (GQ * HD / 2);
              const int g = wi / (HD / 2), d = 2 * (wi % (HD / 2));
              const float inv = 1.0f / stat[g * 2 + 1];
              const uint32_t v = pack2(pv(g * HD + d) * inv, pv(g * HD + d + 1) * inv);
              tput(a.ob + r * a.rep_stride + (size_t)m * (qd / 2) + ((kh * GQ + g) * HD + d) / 2, v, tag);
            }
          } else {
            for (int i = tid; i < GQ * HD * a.rep; i += ANT) {
              const int wi = i % (GQ * HD), r = i / (GQ * HD);
              const float o = pv(wi) / stat[(wi / HD) * 2 + 1];
              tputf(a.ob + r * a.rep_stride + (size_t)m * qd + kh * GQ * HD + wi, o, tag);
            }
          }
        } else {
          for (int i = tid; i < GQ * (HD + 2); i += ANT) {
            const int g = i / (HD + 2), d = i % (HD + 2);
            uint64_t *pp = a.part + ((size_t)(kh * GQ + g) * maxT + t) * (HD + 2);
            float v;
            if (d < HD) {
              const int k = g * HD + d;
              v = pv(k);
            } else {
              v = stat[g * 2 + (d - HD)];
            }
            tputf(pp + d, v, tag);
          }
        }
        __syncthreads();
      }
      if (tracing && tid == 0) {
        uint64_t *tr = a.trace + 8 * (768 + ntr);
        st(tr, (uint64_t)cur.type | ((uint64_t)cur.stack << 8) | ((uint64_t)cur.layer << 16) |
                   ((uint64_t)(cur.step & 0xff) << 24));
        st(tr + 1, t0);
        st(tr + 2, t1);
        st(tr + 3, (uint64_t)wall_clock64());
        ++ntr;
      }
      ev = next_event(a, ev, t);
      if (ev.valid) prep(ev);
    } else if (cur.type == PH_COMB && t == 0) {
      // merge the tile partials of this head's query heads (talker, one row)
      const int ntile = ntiles_at(pos0 + cur.frame);
      uint32_t *buf = (uint32_t *)(smem + L.comb);  // [GQ][ntile][HD + 2]
      const int per = ntile * (HD + 2);
      const bool ok = poll<ANT>(a, GQ * per, tagp, [=](int i) { return buf + i; }, [=](int i) {
        const int g = i / per;
        return a.part + ((size_t)(kh * GQ + g) * maxT) * (HD + 2) + (i - g * per);
      });
      if (!ok) cm.abort = 1;
      __syncthreads();
      if (cm.abort) return;
      const float *pb = (const float *)buf;
      if (a.act_bf16) {
        for (int i = tid; i < GQ * HD / 2; i += ANT) {
          const int g = i / (HD / 2), d = 2 * (i % (HD / 2));
          const float *hp = pb + (size_t)g * ntile * (HD + 2);
          float mx = -INFINITY;
          for (int tt = 0; tt < ntile; ++tt) mx = fmaxf(mx, hp[tt * (HD + 2) + HD]);
          float Ls = 0.f, O0 = 0.f, O1 = 0.f;
          for (int tt = 0; tt < ntile; ++tt) {
            const float w = expf(hp[tt * (HD + 2) + HD] - mx);
            Ls += hp[tt * (HD + 2) + HD + 1] * w;
            O0 += hp[tt * (HD + 2) + d] * w;
            O1 += hp[tt * (HD + 2) + d + 1] * w;
          }
          const uint32_t v = pack2(O0 / Ls, O1 / Ls);
          for (int r = 0; r < a.rep; ++r) tput(a.ob + r * a.rep_stride + ((kh * GQ + g) * HD + d) / 2, v, tag);
        }
      } else {
        for (int i = tid; i < GQ * HD; i += ANT) {
          const int g = i / HD, d = i % HD;
          const float *hp = pb + (size_t)g * ntile * (HD + 2);
          float mx = -INFINITY;
          for (int tt = 0; tt < ntile; ++tt) mx = fmaxf(mx, hp[tt * (HD + 2) + HD]);
          float Ls = 0.f, O = 0.f;
          for (int tt = 0; tt < ntile; ++tt) {
            const float w = expf(hp[tt * (HD + 2) + HD] - mx);
            Ls += hp[tt * (HD + 2) + HD + 1] * w;
            O += hp[tt * (HD + 2) + d] * w;
          }
          for (int r = 0; r < a.rep; ++r) tputf(a.ob + r * a.rep_stride + (size_t)(kh * GQ + g) * HD + d, O / Ls, tag);
        }
      }
      __syncthreads();
    }
    ++seq;
    cur = nxt;
  }
  if (TRC && a.trace && wg == 0 && tid == 0) st(a.trace + 8 * (768 + ntr), (uint64_t)255);
}

// ------------------------------------------------------------ the kernel

template <int WT, int HD, int GQ, bool KVB, bool SMP, bool TRC>
__global__ __launch_bounds__(NTB) void frame_kernel(FrameArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  Common &cm = *reinterpret_cast<Common *>(smem);
  const int tid = threadIdx.x;
  if (tid == 0) {
    cm.abort = 0;
    cm.cbar = 0;
    cm.gdone = 0;
  }
  for (int l = tid; l < a.Lt + a.Lp; l += NT) {
    const LayerDev *src = l < a.Lt ? a.tl + l : a.pl + (l - a.Lt);
    LayerTab &T = cm.lt[l];
    for (int i = 0; i < 7; ++i) { T.w[i] = ld(&src->w[i]); T.sc[i] = ld(&src->sc[i]); }
    T.attn_norm = ld(&src->attn_norm); T.q_norm = ld(&src->q_norm);
    T.k_norm = ld(&src->k_norm); T.mlp_norm = ld(&src->mlp_norm);
  }
  for (int i = tid; i < a.G; i += NT) {
    cm.head_w[i] = ld(a.head_w + i);
    cm.head_sc[i] = a.head_sc ? ld(a.head_sc + i) : nullptr;
  }
  if (tid < PH_END && (int)blockIdx.x >= a.n_attn)
    cm.sh[tid] = share_calc(a, tid, (int)blockIdx.x - a.n_attn, a.nwg - a.n_attn);
  __syncthreads();
  if ((int)blockIdx.x < a.n_attn) {
    if (tid < ANT) attn_role<HD, GQ, KVB, TRC>(a, smem);  // the other waves end here
  } else {
    gemv_role<WT, SMP, TRC>(a, smem);
  }
}

// (weights, head dim, GQA group, bf16 ring) combinations instantiated
#define QT_FRAME_VARIANTS(X) \
  X(W_F32, 64, 2, false) X(W_BF16, 128, 2, true) X(W_Q8, 128, 2, true) X(W_Q4, 128, 2, true)

}  // namespace

// The persistent kernel's exchange words and error flag for callers that
// cannot allocate (qt_decode_frame_noalloc): one array per device, held until
// the process ends.  In host code its name is only a stand-in for the device
// symbol; the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kFrameScratchBytes];

hipError_t frame_scratch_address(void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

bool frame_variant_supported(int wt, int hd, int g, int kvb) {
#define X(W, HD_, G_, K_) if (wt == W && hd == HD_ && g == G_ && (kvb != 0) == K_) return true;
  QT_FRAME_VARIANTS(X)
#undef X
  return false;
}

bool frame_plan(FrameArgs &a, int max_pos, int lds_limit, const char **why) {
  const bool blocked = a.wt == W_Q8 || a.wt == W_Q4;
  const int qd = a.nq * a.hd;
  a.tile = TILE;
  a.max_tiles = a.P / TILE;
  if (a.P % TILE) { *why = "talker positions not a multiple of 256"; return false; }
  if (a.hd * (a.kv_bf16 ? 2 : 4) != 256) { *why = "K/V rows must be 256 bytes"; return false; }
  if (a.H > 2 * NT * HPAIR || a.H % 256) {
    *why = "hidden width above 1920 or not a multiple of 256";
    return false;
  }
  if (a.Lt + a.Lp > MAXLAYERS || a.G > MAXHEADS) { *why = "too many layers or codebooks"; return false; }
  if (a.nwg > 1024) { *why = "more than 1024 workgroups"; return false; }
  if (a.rep < 1 || a.rep > 32) { *why = "exchange copies outside 1..32"; return false; }
  // GEMV rows held in registers per item: hidden-wide rows (gate/up pairs,
  // heads) up to 2 compute blocks (q8, q4: 1), the O and down rows up to 6
  // (q8, q4: 4)
  if (a.H % block_weights(a.wt) || qd % block_weights(a.wt) || a.F % block_weights(a.wt) ||
      row_blocks(a.wt, a.H) > nb_hidden(a.wt) || row_blocks(a.wt, qd) > nb_wide(a.wt) ||
      row_blocks(a.wt, a.F) > nb_wide(a.wt)) {
    *why = "GEMV rows too wide";
    return false;
  }
  a.n_attn = a.nkv * (max_pos / TILE + 1);
  const int NG = a.nwg - a.n_attn;
  if (NG < 16) { *why = "too few GEMV workgroups"; return false; }
  const int NK[5][3] = {{qd + 2 * a.nkv * a.hd, a.H, 1}, {a.H, qd, 1}, {a.F, a.H, 2}, {a.H, a.F, 1}, {a.Vc, a.H, 1}};
  int slot = 0;
  for (int i = 0; i < 5; ++i) {
    const int N = NK[i][0], K = NK[i][1], nm = NK[i][2];
    if (K % block_weights(a.wt) || N % 2) { *why = "GEMV width not a whole number of compute blocks"; return false; }
    if (K > 3072) { *why = "GEMV width above 3072"; return false; }
    const int g = nm;  // gate/up (nm = 2) rows go in pairs
    const int R = g * ((N / g + NG - 1) / NG);
    if (R * nm > MAXR) { *why = "too many rows per workgroup"; return false; }
    int b = R * nm * slot_rowb(a.wt, K);
    if (blocked) b += (int)up1k((uint32_t)(R * nm * (K / 16)));
    if (i == 0 || i == 2 || i == 4) b += (int)up1k((uint32_t)(a.H * (a.tab_bf16 ? 2 : 4)));
    slot = imax(slot, (int)up1k((uint32_t)b));
  }
  a.slot_bytes = slot;
  a.two_slots = 1;
  Lds L = lds_layout(a);
  if ((int)L.g_end > lds_limit) {
    a.two_slots = 0;
    L = lds_layout(a);
  }
  a.lds_bytes = (int)(L.g_end > L.a_end ? L.g_end : L.a_end);
  if (a.lds_bytes > lds_limit) { *why = "LDS plan above the device limit"; return false; }
  return true;
}

// The kernel instantiation of a plan (null if none): sampled or greedy
// heads, with or without phase stamps.
static const void *frame_fn(const FrameArgs &a, bool smp, bool trc) {
  const int g = a.nq / a.nkv;
#define X2(W, HD_, G_, K_, S_, T_)                                                                     \
  if (a.wt == W && a.hd == HD_ && g == G_ && (a.kv_bf16 != 0) == K_ && smp == S_ && trc == T_) \
    return (const void *)frame_kernel<W, HD_, G_, K_, S_, T_>;
#define X1(W, HD_, G_, K_, S_) X2(W, HD_, G_, K_, S_, false) X2(W, HD_, G_, K_, S_, true)
#define X(W, HD_, G_, K_) X1(W, HD_, G_, K_, false) X1(W, HD_, G_, K_, true)
  QT_FRAME_VARIANTS(X)
#undef X
#undef X1
#undef X2
  return nullptr;
}

bool frame_coresident(const FrameArgs &a, int ncu) {
  for (const int v : {0, 1, 2, 3}) {
    const void *fn = frame_fn(a, v & 1, v >> 1);
    int per_cu = 0;
    if (!fn || hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, a.lds_bytes) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NTB, a.lds_bytes) != hipSuccess ||
        (long long)per_cu * ncu < a.nwg)
      return false;
  }
  return true;
}

hipError_t launch_frame_kernel(const FrameArgs &a, hipStream_t s) {
  const void *fn = frame_fn(a, a.inv_temp != 0.f, a.trace != nullptr);
  if (!fn) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, a.lds_bytes);
  if (e != hipSuccess) return e;
  FrameArgs arg = a;
  void *params[] = {&arg};
  // every workgroup waits on the others' exchange words: they must all be
  // resident together, which a cooperative launch guarantees (or refuses)
  return hipLaunchCooperativeKernel(fn, dim3(a.nwg), dim3(NTB), params, (unsigned)a.lds_bytes, s);
}

}  // namespace qtk
