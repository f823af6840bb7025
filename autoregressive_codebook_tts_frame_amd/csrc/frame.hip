// frame.hip -- persistent frame kernel for one stream (gfx950, wave64).
//
// The frame is a chain of dependent phases: per code-predictor micro-step
// ([QT-log] per-layer K/V ring entry: a 2-row prefill then 14 single-row
// decodes) and per talker step, each layer is QKV -> attention -> O (+residual)
// -> gate/up (+SiLU-mul) -> down (+residual), then a head whose argmax picks
// the next code ([QT-tests] fused codec mode entry: in-graph sampler).  A
// kernel launch per phase costs more than the phase's own HBM traffic, the
// failure mode [MC-opt] (closing paragraph) reports for its engine, so one
// launch runs every phase of n frames:
//
//  * Every workgroup walks the same schedule.  A phase's outputs are 64-bit
//    words (tag | value) written and read at agent scope; a consumer spins on
//    the words it needs until their tag is the producing phase's, so no
//    separate barrier or fence is needed.  Every wait is bounded: a timed-out
//    wait raises a device error flag and the kernel drains.
//  * Weight slices are prefetched into registers: right after a phase has its
//    inputs, each lane issues the 16-byte loads of the next phase's slice, so
//    the HBM stream overlaps the next exchange.
//  * The argmax of a head is reduced redundantly by every workgroup from the
//    workgroups' partial maxima, so every workgroup knows every code and builds
//    the next input row (a code-table row, or the talker's 17-row gather-sum,
//    [QT-log] AR inputs entry) itself.
//  * The attention of one (KV head, 256-position tile) always runs on the same
//    workgroup, so K/V rows a workgroup writes into the ring ([QT-log] set_rows
//    entry) are only ever read back by that workgroup.
#include <math.h>

#include "frame.h"
#include "kernels.h"

namespace qtk {
namespace {

constexpr int NT = 256;
constexpr int MAXC = 12;    // 16-byte weight chunks per lane per phase
constexpr int KMAX = 3072;  // longest activation row
constexpr int MAXLAYERS = 40;  // talker + predictor layers held in the LDS weight table
constexpr int MAXHEADS = 32;
constexpr int PER = KMAX / NT;
constexpr uint32_t SPIN_LIMIT = 1u << 21;

enum { PH_QKV = 0, PH_ATTN, PH_COMB, PH_O, PH_GU, PH_D, PH_HEAD, PH_END };

struct Ph {
  int type, stack, layer, step, frame;  // stack 0 predictor, 1 talker; step = micro-step j
};

// Every global access goes through a global-address-space pointer: pointers
// read out of the argument struct would otherwise be flat, and flat loads
// also count against the LDS wait counter, which would make every LDS access
// wait for the in-flight weight prefetch.
#define GAS __attribute__((address_space(1)))
#define LAS __attribute__((address_space(3)))
template <class T> __device__ __forceinline__ GAS T *gp(T *p) { return (GAS T *)p; }
template <class T> __device__ __forceinline__ const GAS T *gp(const T *p) { return (const GAS T *)p; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return __uint_as_float((u | ((u & 0x7fffffu) ? 0x400000u : 0u)) & 0xffff0000u);
  u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint16_t bf16_bits(float f) { return (uint16_t)(__float_as_uint(bf16_rne(f)) >> 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
__device__ __forceinline__ float tab_at(const void *p, int bf16, size_t i) {
  return bf16 ? __uint_as_float((uint32_t)gp((const uint16_t *)p)[i] << 16) : gp((const float *)p)[i];
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// phase tags run on across launches (tag_base advances per launch), so a tag
// is never reused while a buffer could still hold it
__device__ __forceinline__ uint32_t mktag(uint32_t base, uint32_t seq) { return base + seq; }
__device__ __forceinline__ void tput(uint64_t *p, float v, uint32_t tag) {
  __hip_atomic_store(gp(p), ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void tput_u(uint64_t *p, uint32_t v, uint32_t tag) {
  __hip_atomic_store(gp(p), ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tget(const uint64_t *p) {
  return __hip_atomic_load(gp(const_cast<uint64_t *>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int err_get(const int32_t *e) {
  return __hip_atomic_load(gp(const_cast<int32_t *>(e)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void err_set(int32_t *e) {
  __hip_atomic_store(gp(e), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T> __device__ __forceinline__ T ld(const T *p) { return *gp(p); }
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <> __device__ __forceinline__ uint4 ld<uint4>(const uint4 *p) {
  const u32x4 v = *gp((const u32x4 *)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <class T> __device__ __forceinline__ void st(T *p, T v) { *gp(p) = v; }

// Weight pointers of every layer and head, copied into LDS at kernel start:
// computing a weight address must not wait on a vector-memory load, because
// that wait would also cover (in order) the prefetch loads already in flight.
struct LayerTab {
  const void *w[7];
  const uint16_t *sc[7];
  const void *attn_norm, *q_norm, *k_norm, *mlp_norm;
};

struct Shared {
  // next phase's weight slice, loaded straight from HBM into LDS (per wave,
  // per chunk, per lane) so it never occupies registers while in flight
  uint4 wbuf[4][MAXC][64];
  uint16_t sbuf[4][MAXC][64];  // q8 block scales of those chunks
  LayerTab lt[MAXLAYERS];  // talker layers then predictor layers
  const void *head_w[MAXHEADS];
  const uint16_t *head_sc[MAXHEADS];
  float x[2][KMAX];   // phase input rows (prologue applied)
  float bridge[KMAX]; // talker final-normed hidden (next frame's predictor row 0)
  float q[4][128], k[2][128], v[2][128];
  float sc[4][256];
  float red[4][8];
  float stat[4][2];
  float res[4][24];   // per wave: reduced GEMV outputs
  float xold[4][8];   // per wave: residual words of its rows
  float amv[4];
  int ami[4];
  int codes[256];     // codes fed to this frame's gathers
  int code;           // resolved argmax
  int abort;
};

// ------------------------------------------------------------ schedule

__device__ __forceinline__ Ph next_phase(const FrameArgs &a, const Ph &p, bool multi_tile) {
  Ph n = p;
  switch (p.type) {
    case PH_QKV: n.type = PH_ATTN; break;
    case PH_ATTN: n.type = (p.stack == 1 && multi_tile) ? PH_COMB : PH_O; break;
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
        else { n.stack = 1; n.step = -1; }
      } else {
        n.stack = 0; n.step = 0; n.frame = p.frame + 1;
        if (n.frame >= a.n_frames) n.type = PH_END;
      }
      break;
    default: n.type = PH_END;
  }
  return n;
}

__device__ __forceinline__ int split_of(int type) {
  switch (type) {
    case PH_QKV: return SP_QKV;
    case PH_O: return SP_O;
    case PH_GU: return SP_GU;
    case PH_D: return SP_D;
    case PH_HEAD: return SP_HEAD;
    default: return -1;
  }
}

__device__ __forceinline__ const LayerTab &tab_of(const FrameArgs &a, const Shared &sh, const Ph &p) {
  return sh.lt[p.stack ? p.layer : a.Lt + p.layer];
}

// weight row (and its q8 scales) of output row n, matrix mat, for phase p
__device__ __forceinline__ void row_of(const FrameArgs &a, const Shared &sh, const Ph &p, int n, int mat,
                                       int K, const uint8_t *&w, const uint16_t *&sc) {
  const size_t esz = a.wt == W_F32 ? 4 : (a.wt == W_BF16 ? 2 : 1);
  const LayerTab &T = tab_of(a, sh, p);
  int which = 0, r = n;
  const int qd = a.nq * a.hd, kd = a.nkv * a.hd;
  switch (p.type) {
    case PH_QKV:
      if (n < qd) which = LW_Q;
      else if (n < qd + kd) { which = LW_K; r = n - qd; }
      else { which = LW_V; r = n - qd - kd; }
      break;
    case PH_O: which = LW_O; break;
    case PH_GU: which = mat ? LW_U : LW_G; break;
    case PH_D: which = LW_D; break;
    default: {  // head
      const int hi = p.stack ? 0 : 1 + p.step;
      w = (const uint8_t *)sh.head_w[hi] + (size_t)n * K * esz;
      sc = sh.head_sc[hi] ? sh.head_sc[hi] + (size_t)n * (K / 32) : nullptr;
      return;
    }
  }
  w = (const uint8_t *)T.w[which] + (size_t)r * K * esz;
  sc = T.sc[which] ? T.sc[which] + (size_t)r * (K / 32) : nullptr;
}

__device__ __forceinline__ void phase_nk(const FrameArgs &a, int type, int &N, int &K) {
  const int qd = a.nq * a.hd;
  switch (type) {
    case PH_QKV: N = qd + 2 * a.nkv * a.hd; K = a.H; break;
    case PH_O: N = a.H; K = qd; break;
    case PH_GU: N = a.F; K = a.H; break;
    case PH_D: N = a.H; K = a.F; break;
    default: N = a.Vc; K = a.H; break;
  }
}

// ------------------------------------------------------------ GEMV pieces

template <int WT> struct CHK_;
template <> struct CHK_<W_F32> { static constexpr int v = 4; };
template <> struct CHK_<W_BF16> { static constexpr int v = 8; };
template <> struct CHK_<W_Q8> { static constexpr int v = 16; };

template <int WT, int RW, int NM, int CPL>
__device__ __forceinline__ void prefetch_t(const FrameArgs &a, Shared &sh, const Ph &p, int gw, int lane) {
  constexpr int CH = CHK_<WT>::v;
  const int wave = gw & 3;
  int N, K;
  phase_nk(a, p.type, N, K);
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int n = gw * RW + r;  // uniform across the wave
    if (n >= N) continue;
#pragma unroll
    for (int mat = 0; mat < NM; ++mat) {
      const uint8_t *w;
      const uint16_t *sc;
      row_of(a, sh, p, n, mat, K, w, sc);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int i = (r * NM + mat) * CPL + c;
        const int kc = c * 64 + lane;
        // lane l's 16 bytes land at wbuf[wave][i][l]
        __builtin_amdgcn_global_load_lds((const GAS void *)(w + (size_t)kc * 16), (LAS void *)&sh.wbuf[wave][i][0], 16, 0, 0);
        if constexpr (WT == W_Q8)
          __builtin_amdgcn_global_load_lds((const GAS void *)(sc + kc * CH / 32), (LAS void *)&sh.sbuf[wave][i][0], 2, 0, 0);
      }
    }
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x), c, false);
}
// two int8 (bytes b, b+1 of w) as a bf16 pair (exact: |q| <= 127)
__device__ __forceinline__ uint32_t i8pair_bf16(uint32_t w, int b) {
  const float lo = (float)(int8_t)(w >> (8 * b)), hi = (float)(int8_t)(w >> (8 * b + 8));
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// bf16 / q8 weights: the operand row is packed bf16 in LDS (xb), one dot2
// per weight pair; f32 weights keep the float path
template <int WT>
__device__ __forceinline__ float chunk_dot2(const uint4 w, const uint32_t *xb, uint32_t s16) {
  if constexpr (WT == W_BF16) {
    const uint4 x = *(const uint4 *)xb;
    float s = dot2(w.x, x.x, 0.f);
    s = dot2(w.y, x.y, s);
    s = dot2(w.z, x.z, s);
    s = dot2(w.w, x.w, s);
    return s;
  } else {
    const uint4 x0 = *(const uint4 *)xb, x1 = *(const uint4 *)(xb + 4);
    float s = dot2(i8pair_bf16(w.x, 0), x0.x, 0.f);
    s = dot2(i8pair_bf16(w.x, 2), x0.y, s);
    s = dot2(i8pair_bf16(w.y, 0), x0.z, s);
    s = dot2(i8pair_bf16(w.y, 2), x0.w, s);
    s = dot2(i8pair_bf16(w.z, 0), x1.x, s);
    s = dot2(i8pair_bf16(w.z, 2), x1.y, s);
    s = dot2(i8pair_bf16(w.w, 0), x1.z, s);
    s = dot2(i8pair_bf16(w.w, 2), x1.w, s);
    return s * f16_to_f32(s16);
  }
}

template <int WT>
__device__ __forceinline__ float chunk_dot(const uint4 w, const float *x, uint32_t s16) {
  if constexpr (WT == W_F32) {
    const float4 xv = *(const float4 *)x;
    return __uint_as_float(w.x) * xv.x + __uint_as_float(w.y) * xv.y + __uint_as_float(w.z) * xv.z +
           __uint_as_float(w.w) * xv.w;
  } else if constexpr (WT == W_BF16) {
    const float4 x0 = *(const float4 *)x, x1 = *(const float4 *)(x + 4);
    float s = bf16_lo(w.x) * x0.x;
    s += bf16_hi(w.x) * x0.y;
    s += bf16_lo(w.y) * x0.z;
    s += bf16_hi(w.y) * x0.w;
    s += bf16_lo(w.z) * x1.x;
    s += bf16_hi(w.z) * x1.y;
    s += bf16_lo(w.w) * x1.z;
    s += bf16_hi(w.w) * x1.w;
    return s;
  } else {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 xv = *(const float4 *)(x + 4 * i);
      s += (float)(int8_t)(ws[i]) * xv.x;
      s += (float)(int8_t)(ws[i] >> 8) * xv.y;
      s += (float)(int8_t)(ws[i] >> 16) * xv.z;
      s += (float)(int8_t)(ws[i] >> 24) * xv.w;
    }
    return s * f16_to_f32(s16);
  }
}

// reduced results -> sh.res[wave][(r * NM + mat) * M + m] (all lanes hold them)
template <int WT, int RW, int NM, int CPL, int M>
__device__ __forceinline__ void gemv_t(Shared &sh, int lane, int wave) {
  constexpr int CH = CHK_<WT>::v;
  float acc[RW * NM][M];
#pragma unroll
  for (int i = 0; i < RW * NM; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.f;
#pragma unroll
  for (int rm = 0; rm < RW * NM; ++rm)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int i = rm * CPL + c;
      const int k0 = (c * 64 + lane) * CH;
      const uint4 wv = sh.wbuf[wave][i][lane];
      const uint32_t sv = WT == W_Q8 ? (uint32_t)sh.sbuf[wave][i][lane] : 0u;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if constexpr (WT == W_F32) acc[rm][m] += chunk_dot<WT>(wv, &sh.x[m][k0], sv);
        else acc[rm][m] += chunk_dot2<WT>(wv, (const uint32_t *)&sh.x[m][0] + k0 / 2, sv);
      }
      // keep one chunk's operands live at a time: hoisting every chunk's LDS
      // reads would spill the prefetched weights of the next phase
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
  for (int rm = 0; rm < RW * NM; ++rm)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float v = wave_sum(acc[rm][m]);
      if (lane == 0) sh.res[wave][rm * M + m] = v;
    }
}

#define QT_SPLITS(X)                                                                     \
  X(W_F32, 1, 1, 1) X(W_F32, 1, 2, 1) X(W_F32, 1, 1, 3)                                  \
  X(W_BF16, 4, 1, 2) X(W_BF16, 1, 1, 4) X(W_BF16, 3, 2, 2) X(W_BF16, 1, 1, 6) X(W_BF16, 2, 1, 2) \
  X(W_Q8, 4, 1, 1) X(W_Q8, 1, 1, 2) X(W_Q8, 3, 2, 1) X(W_Q8, 1, 1, 3) X(W_Q8, 2, 1, 1)

template <int WT>
__device__ __forceinline__ void prefetch_any(const FrameArgs &a, Shared &sh, const Ph &p, int gw, int lane) {
  const int si = split_of(p.type);
  if (si < 0) return;
  const Split sp = a.split[si];
#define X(W, R, N, C) \
  if (WT == W && sp.rw == R && sp.nmat == N && sp.cpl == C) { prefetch_t<W, R, N, C>(a, sh, p, gw, lane); return; }
  QT_SPLITS(X)
#undef X
}

template <int WT>
__device__ __forceinline__ void gemv_any(const FrameArgs &a, int type, int M, Shared &sh, int lane, int wave) {
  const Split sp = a.split[split_of(type)];
#define X(W, R, N, C)                                                                     \
  if (WT == W && sp.rw == R && sp.nmat == N && sp.cpl == C) {                            \
    if (M == 1) gemv_t<W, R, N, C, 1>(sh, lane, wave);                                    \
    else gemv_t<W, R, N, C, 2>(sh, lane, wave);                                           \
    return;                                                                              \
  }
  QT_SPLITS(X)
#undef X
}

// ------------------------------------------------------------ exchange

// n tagged words src[0..n) with tag -> dst (LDS floats); all threads; false on timeout
__device__ __forceinline__ bool acquire(const FrameArgs &a, const uint64_t *src, int n, uint32_t tag, float *dst) {
  uint64_t v[PER];
  uint32_t pend = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < n) {
      v[k] = tget(src + i);
      pend |= 1u << k;
    }
  }
  for (uint32_t spins = 0;; ++spins) {
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if ((pend >> k) & 1u) {
        if ((uint32_t)(v[k] >> 32) == tag) {
          dst[threadIdx.x + k * NT] = __uint_as_float((uint32_t)v[k]);
          pend &= ~(1u << k);
        }
      }
    if (!pend) return true;
    if (spins > SPIN_LIMIT || ((spins & 1023u) == 1023u && err_get(a.err))) {
      err_set(a.err);
      return false;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if ((pend >> k) & 1u) v[k] = tget(src + threadIdx.x + k * NT);
  }
}

// one tagged word (single lane); false on timeout
__device__ __forceinline__ bool acquire1(const FrameArgs &a, const uint64_t *src, uint32_t tag, uint32_t &out) {
  uint64_t v = tget(src);
  for (uint32_t spins = 0; (uint32_t)(v >> 32) != tag; ++spins) {
    if (spins > SPIN_LIMIT || ((spins & 1023u) == 1023u && err_get(a.err))) {
      err_set(a.err);
      return false;
    }
    v = tget(src);
  }
  out = (uint32_t)v;
  return true;
}

// block-wide sum of per-thread values (fixed order)
__device__ __forceinline__ float block_sum(Shared &sh, float v, int slot) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh.red[wave][slot] = v;
  __syncthreads();
  return (sh.red[0][slot] + sh.red[1][slot]) + (sh.red[2][slot] + sh.red[3][slot]);
}

// RMSNorm rows of sh.x in place: x <- act(x / rms(x) * g); keep optional f32 copy
__device__ __forceinline__ void norm_rows(const FrameArgs &a, Shared &sh, int M, int K, const void *gain, float *keep) {
  for (int m = 0; m < M; ++m) {
    float s = 0.f;
    for (int i = threadIdx.x; i < K; i += NT) s += sh.x[m][i] * sh.x[m][i];
    s = block_sum(sh, s, m);
    const float r = 1.0f / sqrtf(s / (float)K + a.eps);
    for (int i = threadIdx.x; i < K; i += NT) {
      const float y = sh.x[m][i] * r * tab_at(gain, a.tab_bf16, i);
      if (keep) keep[i] = y;
      sh.x[m][i] = a.act_bf16 ? bf16_rne(y) : y;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void act_rows(const FrameArgs &a, Shared &sh, int M, int K) {
  if (a.act_bf16)
    for (int m = 0; m < M; ++m)
      for (int i = threadIdx.x; i < K; i += NT) sh.x[m][i] = bf16_rne(sh.x[m][i]);
  __syncthreads();
}

// ------------------------------------------------------------ attention

// Ring rows are read and written as 8-byte words at agent scope (4 bf16 or 2
// f32 per word): the code-predictor cache is rewritten every frame by the same
// workgroup that reads it, and these accesses never see a stale cached line.
template <bool KVB>
__device__ __forceinline__ void unpack8(uint64_t w, float *v) {
  if constexpr (KVB) {
    v[0] = __uint_as_float((uint32_t)(w << 16) & 0xffff0000u);
    v[1] = __uint_as_float((uint32_t)w & 0xffff0000u);
    v[2] = __uint_as_float((uint32_t)(w >> 16) & 0xffff0000u);
    v[3] = __uint_as_float((uint32_t)(w >> 32) & 0xffff0000u);
  } else {
    v[0] = __uint_as_float((uint32_t)w);
    v[1] = __uint_as_float((uint32_t)(w >> 32));
  }
}
template <bool KVB>
__device__ __forceinline__ uint64_t pack8(const float *v) {
  if constexpr (KVB)
    return (uint64_t)bf16_bits(v[0]) | ((uint64_t)bf16_bits(v[1]) << 16) |
           ((uint64_t)bf16_bits(v[2]) << 32) | ((uint64_t)bf16_bits(v[3]) << 48);
  else
    return (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32);
}
__device__ __forceinline__ void ring_put(uint64_t *p, uint64_t v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One (KV head kh, tile t) attention unit for rows at positions pos0, pos1
// (M <= 2).  HD head dim, G query heads per KV head, KVB bf16 ring.
template <int HD, int G, bool KVB>
__device__ __forceinline__ bool attention_unit(const FrameArgs &a, Shared &sh, const Ph &p, int kh,
                                               int t, int M, int pos0, int pos1, uint32_t tag_in,
                                               uint32_t tag_out, int ntiles, int tile) {
  constexpr int VPW = KVB ? 4 : 2;   // values per 8-byte word
  constexpr int WPR = HD / VPW;      // words per ring row
  constexpr int NGRP = NT / WPR;     // position groups of the P.V loop
  constexpr int HALF = HD / 2;
  const int qd = a.nq * HD, kd = a.nkv * HD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = p.stack ? a.P : a.Q;
  const int64_t kvs_w = (p.stack ? a.t_kv_stride : a.p_kv_stride) / VPW;
  uint64_t *ring = (uint64_t *)((p.stack ? a.ring_t : a.ring_p) +
                                (size_t)p.layer * (p.stack ? a.t_layer_stride : a.p_layer_stride) * (KVB ? 2 : 4));
  const size_t head_w = (size_t)kh * P * WPR;
  const LayerTab &T = tab_of(a, sh, p);
  const void *qn = T.q_norm, *kn = T.k_norm;
  const int nqkv = qd + 2 * kd;
  for (int m = 0; m < M; ++m) {
    const int pm = m ? pos1 : pos0;
    const int j0 = t * tile;
    if (j0 > pm) continue;  // uniform across the block
    const int jn = min(tile, pm + 1 - j0);
    // q (G heads), k, v of this KV head, row m
    const uint64_t *row = a.qkvb + (size_t)m * nqkv;
    bool ok = acquire(a, row + kh * G * HD, G * HD, tag_in, &sh.sc[0][0]);
    ok = ok && acquire(a, row + qd + kh * HD, HD, tag_in, &sh.sc[2][0]);
    ok = ok && acquire(a, row + qd + kd + kh * HD, HD, tag_in, &sh.sc[3][0]);
    if (!ok) sh.abort = 1;
    __syncthreads();
    if (sh.abort) return false;
    // q/k norm + RoPE: wave w < G handles q head w, wave G the k head; lanes own pairs
    if (wave <= G) {
      const float *src = wave < G ? &sh.sc[0][wave * HD] : &sh.sc[2][0];
      const void *gain = wave < G ? qn : kn;
      const bool act = lane < HALF;
      const float x0 = act ? src[lane] : 0.f, x1 = act ? src[lane + HALF] : 0.f;
      const float s = wave_sum(x0 * x0 + x1 * x1);
      const float rv = 1.0f / sqrtf(s / (float)HD + a.eps);
      if (act) {
        const float y0 = x0 * rv * tab_at(gain, a.tab_bf16, lane);
        const float y1 = x1 * rv * tab_at(gain, a.tab_bf16, lane + HALF);
        const float c = ld(a.rope_cos + (size_t)pm * HALF + lane), sn = ld(a.rope_sin + (size_t)pm * HALF + lane);
        const float o0 = y0 * c - y1 * sn, o1 = y1 * c + y0 * sn;
        float *dst = wave < G ? sh.q[wave] : sh.k[0];
        dst[lane] = o0;
        dst[lane + HALF] = o1;
      }
    }
    for (int i = tid; i < HD; i += NT) sh.v[0][i] = sh.sc[3][i];
    __syncthreads();
    // the tile holding this row's position writes its K/V rows (set_rows)
    if (pm < j0 + tile && tid < 2 * WPR) {
      const int wi = tid % WPR;
      const bool isv = tid >= WPR;
      ring_put(ring + head_w + (isv ? kvs_w : 0) + (size_t)pm * WPR + wi,
               pack8<KVB>((isv ? sh.v[0] : sh.k[0]) + wi * VPW));
    }
    __syncthreads();
    // scores: one thread per position of the tile; positions past pm are
    // excluded by select and their rows never read
    if (tid < tile) {
      if (tid < jn) {
        const uint64_t *kr = ring + head_w + (size_t)(j0 + tid) * WPR;
        uint64_t kw[WPR];
#pragma unroll
        for (int wi = 0; wi < WPR; ++wi) kw[wi] = tget(kr + wi);
        float s[G];
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = 0.f;
#pragma unroll
        for (int wi = 0; wi < WPR; ++wi) {
          float kv[4];
          unpack8<KVB>(kw[wi], kv);
#pragma unroll
          for (int i = 0; i < VPW; ++i)
#pragma unroll
            for (int g = 0; g < G; ++g) s[g] += sh.q[g][wi * VPW + i] * kv[i];
        }
#pragma unroll
        for (int g = 0; g < G; ++g) sh.sc[g][tid] = s[g] * a.scale;
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) sh.sc[g][tid] = -INFINITY;
      }
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float v = tid < tile ? sh.sc[g][tid] : -INFINITY;
      v = wave_max(v);
      if (lane == 0) sh.red[wave][g] = v;
    }
    __syncthreads();
    if (tid < G) sh.stat[tid][0] = fmaxf(fmaxf(sh.red[0][tid], sh.red[1][tid]), fmaxf(sh.red[2][tid], sh.red[3][tid]));
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float e = 0.f;
      if (tid < jn) e = expf(sh.sc[g][tid] - sh.stat[g][0]);
      if (tid < tile) sh.sc[g][tid] = e;
      e = wave_sum(e);
      if (lane == 0) sh.red[wave][4 + g] = e;
    }
    __syncthreads();
    if (tid < G) sh.stat[tid][1] = (sh.red[0][4 + tid] + sh.red[1][4 + tid]) + (sh.red[2][4 + tid] + sh.red[3][4 + tid]);
    // P.V: thread (group, word) accumulates positions j = group, group+NGRP, ...
    {
      const int wi = tid % WPR, grp = tid / WPR;
      float acc[G][VPW];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < VPW; ++i) acc[g][i] = 0.f;
      const uint64_t *vr = ring + head_w + kvs_w + (size_t)j0 * WPR + wi;
      int j = grp;
      for (; j + 3 * NGRP < jn; j += 4 * NGRP) {
        uint64_t vw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) vw[u] = tget(vr + (size_t)(j + u * NGRP) * WPR);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float vv[4];
          unpack8<KVB>(vw[u], vv);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float e = sh.sc[g][j + u * NGRP];
#pragma unroll
            for (int i = 0; i < VPW; ++i) acc[g][i] += e * vv[i];
          }
        }
      }
      for (; j < jn; j += NGRP) {
        float vv[4];
        unpack8<KVB>(tget(vr + (size_t)j * WPR), vv);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float e = sh.sc[g][j];
#pragma unroll
          for (int i = 0; i < VPW; ++i) acc[g][i] += e * vv[i];
        }
      }
      // partials by group -> LDS (sh.x as scratch: [grp][g][HD])
      float *scr = &sh.x[0][0];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < VPW; ++i) scr[((size_t)grp * G + g) * HD + wi * VPW + i] = acc[g][i];
    }
    __syncthreads();
    if (tid < G * HD) {
      const int g = tid / HD, d = tid % HD;
      const float *scr = &sh.x[0][0];
      float acc = 0.f;
#pragma unroll
      for (int grp = 0; grp < NGRP; ++grp) acc += scr[((size_t)grp * G + g) * HD + d];
      const int h = kh * G + g;
      if (ntiles == 1) {
        tput(a.ob + (size_t)m * qd + (size_t)h * HD + d, acc / sh.stat[g][1], tag_out);
      } else {
        uint64_t *pp = a.part + ((size_t)h * (a.P / 256) + t) * (HD + 2);
        tput(pp + d, acc, tag_out);
        if (d == 0) {
          tput(pp + HD, sh.stat[g][0], tag_out);
          tput(pp + HD + 1, sh.stat[g][1], tag_out);
        }
      }
    }
    __syncthreads();
  }
  return true;
}

// merge the tile partials of query head h (talker, one row)
__device__ __forceinline__ bool combine_unit(const FrameArgs &a, Shared &sh, int h, int ntiles, uint32_t tag_in,
                             uint32_t tag_out) {
  const int hd = a.hd, tid = threadIdx.x;
  const uint64_t *base = a.part + (size_t)h * (a.P / 256) * (hd + 2);
  // stage all partials: ntiles * (hd + 2) words <= 16 * 130
  const int n = ntiles * (hd + 2);
  if (!acquire(a, base, n, tag_in, &sh.x[0][0])) sh.abort = 1;
  __syncthreads();
  if (sh.abort) return false;
  if (tid < hd) {
    float mx = -INFINITY;
    for (int t = 0; t < ntiles; ++t) mx = fmaxf(mx, sh.x[0][t * (hd + 2) + hd]);
    float Lsum = 0.f, O = 0.f;
    for (int t = 0; t < ntiles; ++t) {
      const float w = expf(sh.x[0][t * (hd + 2) + hd] - mx);
      Lsum += sh.x[0][t * (hd + 2) + hd + 1] * w;
      O += sh.x[0][t * (hd + 2) + tid] * w;
    }
    tput(a.ob + (size_t)h * hd + tid, O / Lsum, tag_out);
  }
  __syncthreads();
  return true;
}

// ------------------------------------------------------------ the kernel

template <int WT, int HD, int GQ, bool KVB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void frame_kernel(FrameArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Shared &sh = *reinterpret_cast<Shared *>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wg = blockIdx.x;
  const int gw = wg * 4 + wave;
  const int H = a.H, qd = a.nq * a.hd;
  const int force = ld(a.ctl + 1);
  const int tiles_max = a.P / 256;

  int pos = ld(a.pos);
  int c0 = ld(a.c0);
  if (tid == 0) sh.abort = 0;
  for (int l = tid; l < a.Lt + a.Lp; l += NT) {
    const LayerDev *src = l < a.Lt ? a.tl + l : a.pl + (l - a.Lt);
    LayerTab &T = sh.lt[l];
    for (int i = 0; i < 7; ++i) { T.w[i] = ld(&src->w[i]); T.sc[i] = ld(&src->sc[i]); }
    T.attn_norm = ld(&src->attn_norm); T.q_norm = ld(&src->q_norm);
    T.k_norm = ld(&src->k_norm); T.mlp_norm = ld(&src->mlp_norm);
  }
  for (int i = tid; i < a.G; i += NT) {
    sh.head_w[i] = ld(a.head_w + i);
    sh.head_sc[i] = a.head_sc ? ld(a.head_sc + i) : nullptr;
  }
  for (int i = tid; i < H; i += NT) sh.bridge[i] = ld(a.bridge + i);
  __syncthreads();

  uint32_t seq = 1, x_seq = 0;
  // the weight slice of a phase sits in sh.wbuf: a phase consumes it, then
  // loads the next phase's slice there before its stores and the next wait
  __syncthreads();

  Ph cur{PH_QKV, 0, 0, 0, 0};
  bool pending_code = false;     // the previous phase was a head
  int pending_idx = 0;           // code index it decides (0 = next frame's c0)
  prefetch_any<WT>(a, sh, cur, gw, lane);

  int ntr = 0;
  uint64_t t_start = 0;
  while (cur.type != PH_END) {
    const bool tracing = a.trace && wg == 0 && cur.frame == 0 && ntr < 1023;  // [1024][8] words
    if (tracing) t_start = wall_clock64();
    const uint32_t tag = mktag(a.tag_base, seq);
    const uint32_t tag_prev = mktag(a.tag_base, seq - 1);
    const bool multi = ((pos + 256) / 256) > 1;

    // ---- resolve the code picked by the previous head (every workgroup)
    if (pending_code) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int w = tid; w < a.nwg; w += NT) {
        uint32_t v, ix;
        bool ok = acquire1(a, a.amax + 2 * w, tag_prev, v) && acquire1(a, a.amax + 2 * w + 1, tag_prev, ix);
        if (!ok) { sh.abort = 1; break; }
        const float fv = __uint_as_float(v);
        if (fv > bv || (fv == bv && (int)ix < bi)) { bv = fv; bi = (int)ix; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (lane == 0) { sh.amv[wave] = bv; sh.ami[wave] = bi; }
      __syncthreads();
      if (sh.abort) return;
      if (tid == 0) {
        float b2 = sh.amv[0];
        int i2 = sh.ami[0];
        for (int w = 1; w < 4; ++w)
          if (sh.amv[w] > b2 || (sh.amv[w] == b2 && sh.ami[w] < i2)) { b2 = sh.amv[w]; i2 = sh.ami[w]; }
        sh.code = i2 == 0x7fffffff ? 0 : i2;
      }
      __syncthreads();
      const int c = sh.code;
      if (pending_idx == 0) {
        c0 = c;  // next frame's code 0 (the talker's pick)
      } else {
        const int f = cur.frame;  // same frame as the predictor head
        int32_t *ci = a.cin + (size_t)f * a.G + pending_idx;
        if (wg == 0 && tid == 0) {
          st(a.cout + (size_t)f * a.G + pending_idx, c);
          if (!force) st(ci, c);
        }
        if (tid == 0) sh.codes[pending_idx] = force ? ld(ci) : c;
      }
      pending_code = false;
      __syncthreads();
    }

    const int f = cur.frame;
    if (cur.type == PH_END) break;

    // ---- inputs of this phase
    int M = 1;
    bool ok = true;
    int pos0 = 0, pos1 = 0;
    if (cur.stack == 0) {
      if (cur.step == 0) { M = 2; pos0 = 0; pos1 = 1; }
      else pos0 = cur.step + 1;
    } else {
      pos0 = pos;
    }

    if (cur.type == PH_QKV && cur.layer == 0) {
      // build the stack's input rows locally
      if (cur.stack == 0 && cur.step == 0) {
        // frame start: code 0 of the frame, then rows [bridge, E_0[c0]]
        int32_t *ci = a.cin + (size_t)f * a.G;
        if (wg == 0 && tid == 0) {
          st(a.cout + (size_t)f * a.G, c0);
          if (!force) st(ci, c0);
        }
        if (tid == 0) sh.codes[0] = force ? ld(ci) : c0;
        __syncthreads();
        const int cc = sh.codes[0];
        for (int i = tid; i < H; i += NT) {
          sh.x[0][i] = sh.bridge[i];
          sh.x[1][i] = tab_at(a.code_emb, a.tab_bf16, (size_t)cc * H + i);
        }
      } else if (cur.stack == 0) {
        const int cc = sh.codes[cur.step];
        for (int i = tid; i < H; i += NT)
          sh.x[0][i] = tab_at(a.code_emb, a.tab_bf16, ((size_t)cur.step * a.Vc + cc) * H + i);
      } else {
        // talker input: sum of the G code rows + the overlay row, left to right
        const int ov = ld(a.overlay + f);
        for (int i = tid; i < H; i += NT) {
          float acc = 0.f;
          for (int g = 0; g < a.G; ++g)
            acc += tab_at(a.code_emb, a.tab_bf16, ((size_t)g * a.Vc + sh.codes[g]) * H + i);
          acc += tab_at(a.text_emb, a.tab_bf16, (size_t)ov * H + i);
          sh.x[0][i] = acc;
          if (a.dump && wg == 0) st(a.x0_dump + i, acc);
        }
        if (a.dump && wg == 0 && tid <= a.G) st(a.gather_dump + tid, tid < a.G ? sh.codes[tid] : ov);
        if (a.dump && wg == 0 && tid == 0) st(a.tpos_dump, pos);
      }
      __syncthreads();
      // publish the rows for the residual adds: element i by workgroup i % nwg
      for (int m = 0; m < M; ++m)
        for (int i = wg + a.nwg * tid; i < H; i += a.nwg * NT) tput(a.xq + (size_t)m * H + i, sh.x[m][i], tag);
      x_seq = seq;
    } else if (cur.type == PH_QKV || cur.type == PH_GU || cur.type == PH_HEAD) {
      const int mrow = (cur.type == PH_HEAD && cur.stack == 0 && cur.step == 0) ? 1 : 0;
      if (cur.type == PH_HEAD) M = 1;
      for (int m = 0; m < M; ++m)
        ok = ok && acquire(a, a.xq + (size_t)(m + mrow) * H, H, mktag(a.tag_base, x_seq), sh.x[m]);
    } else if (cur.type == PH_O) {
      for (int m = 0; m < M; ++m) ok = ok && acquire(a, a.ob + (size_t)m * qd, qd, tag_prev, sh.x[m]);
    } else if (cur.type == PH_D) {
      for (int m = 0; m < M; ++m) ok = ok && acquire(a, a.zb + (size_t)m * a.F, a.F, tag_prev, sh.x[m]);
    }
    // residual words of this wave's rows
    if (ok && (cur.type == PH_O || cur.type == PH_D)) {
      const Split sp = a.split[split_of(cur.type)];
      if (lane < sp.rw * M) {
        const int r = lane / M, m = lane % M;
        const int n = gw * sp.rw + r;
        if (n < H) {
          uint32_t v;
          if (!acquire1(a, a.xq + (size_t)m * H + n, mktag(a.tag_base, x_seq), v)) ok = false;
          else sh.xold[wave][lane] = __uint_as_float(v);
        }
      }
    }
    if (!ok) sh.abort = 1;
    __syncthreads();
    if (sh.abort) return;

    uint64_t t_in = 0, t_pro = 0, t_w = 0, t_mm = 0;
    if (tracing) t_in = wall_clock64();
    // ---- prologue: norm / operand rounding
    const LayerTab &Lc = tab_of(a, sh, cur);
    if (cur.type == PH_QKV) norm_rows(a, sh, M, H, Lc.attn_norm, nullptr);
    else if (cur.type == PH_GU) norm_rows(a, sh, M, H, Lc.mlp_norm, nullptr);
    else if (cur.type == PH_HEAD) {
      const bool talker = cur.stack == 1;
      norm_rows(a, sh, 1, H, talker ? a.t_norm : a.p_norm, talker ? sh.bridge : nullptr);
      if (talker && wg == 0)
        for (int i = tid; i < H; i += NT) st(a.bridge + i, sh.bridge[i]);
    } else if (cur.type == PH_O) act_rows(a, sh, M, qd);
    else if (cur.type == PH_D) act_rows(a, sh, M, a.F);
    if constexpr (WT != W_F32) {
      // GEMV operand rows -> packed bf16 pairs in place (values are already
      // bf16-rounded, so this is exact)
      if (cur.type != PH_ATTN && cur.type != PH_COMB) {
        int N_, K_;
        phase_nk(a, cur.type, N_, K_);
        const int Mg = cur.type == PH_HEAD ? 1 : M;
        uint32_t pk[2][KMAX / (2 * NT)];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int k = 0; k < KMAX / (2 * NT); ++k) {
            const int pi = tid + k * NT;
            pk[m][k] = 0;
            if (m < Mg && 2 * pi < K_)
              pk[m][k] = (__float_as_uint(sh.x[m][2 * pi]) >> 16) | (__float_as_uint(sh.x[m][2 * pi + 1]) & 0xffff0000u);
          }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int k = 0; k < KMAX / (2 * NT); ++k) {
            const int pi = tid + k * NT;
            if (m < Mg && 2 * pi < K_) ((uint32_t *)&sh.x[m][0])[pi] = pk[m][k];
          }
        __syncthreads();
      }
    }

    if (tracing) t_pro = wall_clock64();
    const Ph nxt = next_phase(a, cur, multi);
    // workgroups with attention work issue the next prefetch after it (their
    // waits for q/k/v would otherwise also wait for the prefetch, in order)
    const bool attn_busy =
        (cur.type == PH_ATTN && wg < a.nkv * (cur.stack ? tiles_max : 1)) || (cur.type == PH_COMB && wg < a.nq);

    // ---- compute + epilogue
    if (attn_busy) {
      // attention first: the next phase's weights are not in flight meanwhile
      if (cur.type == PH_ATTN) {
        const int tile = cur.stack ? 256 : a.Q;
        const int ntiles = cur.stack ? (pos + 256) / 256 : 1;
        const int units = a.nkv * (cur.stack ? tiles_max : 1);
        for (int u = wg; u < units; u += a.nwg) {
          const int kh = cur.stack ? u / tiles_max : u;
          const int t = cur.stack ? u % tiles_max : 0;
          if (!attention_unit<HD, GQ, KVB>(a, sh, cur, kh, t, M, pos0, pos1, tag_prev, tag, ntiles, tile)) return;
        }
      } else {
        const int ntiles = (pos + 256) / 256;
        for (int h = wg; h < a.nq; h += a.nwg)
          if (!combine_unit(a, sh, h, ntiles, tag_prev, tag)) return;
      }
      prefetch_any<WT>(a, sh, nxt, gw, lane);
    } else if (cur.type == PH_ATTN || cur.type == PH_COMB) {
      prefetch_any<WT>(a, sh, nxt, gw, lane);
    }
    if (cur.type != PH_ATTN && cur.type != PH_COMB) {
      int N, K;
      phase_nk(a, cur.type, N, K);
      // the slice's LDS-direct loads count as vector-memory operations: wait
      // for them (long done after the input exchange, which waited in order)
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      if (tracing) t_w = wall_clock64();
      gemv_any<WT>(a, cur.type, M, sh, lane, wave);
      if (tracing) t_mm = wall_clock64();
      // each wave reads back only its own slice, so the next phase's loads
      // may land once this wave's reads are done
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      prefetch_any<WT>(a, sh, nxt, gw, lane);
      const Split sp = a.split[split_of(cur.type)];
      const int nout = sp.rw * M;
      if (cur.type == PH_HEAD) {
        // logits (kept for readback) and this workgroup's partial argmax
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        float *lg = cur.stack ? a.logits_t : a.logits_p + (size_t)cur.step * a.Vc;
        if (lane < sp.rw) {
          const int n = gw * sp.rw + lane;
          if (n < N) {
            bv = sh.res[wave][lane];
            bi = n;
            st(lg + n, bv);
          }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float ov = __shfl_xor(bv, o, 64);
          const int oi = __shfl_xor(bi, o, 64);
          if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        if (lane == 0) { sh.amv[wave] = bv; sh.ami[wave] = bi; }
        __syncthreads();
        if (tid == 0) {
          float b2 = sh.amv[0];
          int i2 = sh.ami[0];
          for (int w = 1; w < 4; ++w)
            if (sh.amv[w] > b2 || (sh.amv[w] == b2 && sh.ami[w] < i2)) { b2 = sh.amv[w]; i2 = sh.ami[w]; }
          tput(a.amax + 2 * wg, b2, tag);
          tput_u(a.amax + 2 * wg + 1, (uint32_t)i2, tag);
        }
        pending_code = true;
        pending_idx = cur.stack ? 0 : cur.step + 1;
        if (cur.stack == 1) {
          if (wg == 0 && tid == 0) st(a.pos, pos + 1);
          pos += 1;
        }
      } else if (lane < nout) {
        const int r = lane / M, m = lane % M;
        const int n = gw * sp.rw + r;
        if (n < N) {
          if (cur.type == PH_QKV) {
            tput(a.qkvb + (size_t)m * N + n, sh.res[wave][r * M + m], tag);
          } else if (cur.type == PH_GU) {
            const float g = sh.res[wave][(r * 2) * M + m], u = sh.res[wave][(r * 2 + 1) * M + m];
            tput(a.zb + (size_t)m * N + n, g / (1.0f + expf(-g)) * u, tag);
          } else {
            const float nv = sh.xold[wave][lane] + sh.res[wave][r * M + m];
            tput(a.xq + (size_t)m * H + n, nv, tag);
            if (cur.type == PH_D && cur.stack == 1 && a.dump)
              st(a.hidden_dump + (size_t)cur.layer * H + n, nv);
          }
        }
      }
      if (cur.type == PH_O || cur.type == PH_D) x_seq = seq;
    }
    __syncthreads();
    if (tracing && tid == 0) {
      uint64_t *tr = a.trace + 8 * ntr;
      st(tr, (uint64_t)cur.type | ((uint64_t)cur.stack << 8) | ((uint64_t)cur.layer << 16) |
                 ((uint64_t)(cur.step & 0xff) << 24));
      st(tr + 1, t_start);
      st(tr + 2, t_in);
      st(tr + 3, (uint64_t)wall_clock64());
      st(tr + 4, t_pro);
      st(tr + 5, t_w);
      st(tr + 6, t_mm);
    }
    if (tracing) ++ntr;
    ++seq;
    cur = nxt;
  }
  if (a.trace && wg == 0 && tid == 0) st(a.trace + 8 * ntr, (uint64_t)255);
  // the code picked by the last talker head becomes the slot's pending code 0
  if (pending_code) {
    const uint32_t tag_prev = mktag(a.tag_base, seq - 1);
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    bool ok = true;
    for (int w = tid; w < a.nwg; w += NT) {
      uint32_t v, ix;
      if (!(acquire1(a, a.amax + 2 * w, tag_prev, v) && acquire1(a, a.amax + 2 * w + 1, tag_prev, ix))) { ok = false; break; }
      const float fv = __uint_as_float(v);
      if (fv > bv || (fv == bv && (int)ix < bi)) { bv = fv; bi = (int)ix; }
    }
    if (!ok) sh.abort = 1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) { sh.amv[wave] = bv; sh.ami[wave] = bi; }
    __syncthreads();
    if (sh.abort) return;
    if (wg == 0 && tid == 0) {
      float b2 = sh.amv[0];
      int i2 = sh.ami[0];
      for (int w = 1; w < 4; ++w)
        if (sh.amv[w] > b2 || (sh.amv[w] == b2 && sh.ami[w] < i2)) { b2 = sh.amv[w]; i2 = sh.ami[w]; }
      st(a.c0, i2 == 0x7fffffff ? 0 : i2);
    }
  }
}

}  // namespace

bool frame_split_supported(int wt, const Split &sp) {
#define X(W, R, N, C) \
  if (wt == W && sp.rw == R && sp.nmat == N && sp.cpl == C) return true;
  QT_SPLITS(X)
#undef X
  return false;
}

// (weights, head dim, GQA group, bf16 ring) combinations instantiated
#define QT_FRAME_VARIANTS(X)                                   \
  X(W_F32, 64, 2, false) X(W_F32, 128, 2, false)               \
  X(W_BF16, 128, 2, true) X(W_BF16, 128, 1, true) X(W_BF16, 64, 2, true) \
  X(W_Q8, 128, 2, true) X(W_Q8, 128, 1, true)

bool frame_variant_supported(int wt, int hd, int g, int kvb) {
#define X(W, HD_, G_, K_) if (wt == W && hd == HD_ && g == G_ && (kvb != 0) == K_) return true;
  QT_FRAME_VARIANTS(X)
#undef X
  return false;
}

size_t frame_lds_bytes() { return sizeof(Shared); }

hipError_t launch_frame_kernel(const FrameArgs &a, hipStream_t s) {
  const int g = a.nq / a.nkv;
#define X(W, HD_, G_, K_)                                                                         \
  if (a.wt == W && a.hd == HD_ && g == G_ && (a.kv_bf16 != 0) == K_) {                          \
    hipError_t e = hipFuncSetAttribute((const void *)frame_kernel<W, HD_, G_, K_>,                \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Shared)); \
    if (e != hipSuccess) return e;                                                               \
    hipLaunchKernelGGL((frame_kernel<W, HD_, G_, K_>), dim3(a.nwg), dim3(NT), sizeof(Shared), s, a); \
    return hipGetLastError();                                                                    \
  }
  QT_FRAME_VARIANTS(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace qtk
