// kernels.hip -- gfx950 kernels of the per-frame decode step.
//
// Wave64 throughout.  Weight matrices are streamed once per launch with
// 128-bit loads, each lane owning 16-byte chunks along K; activations are
// read in f32 and turned into the matmul operand in registers (optional
// RMSNorm prologue, optional bf16 RNE rounding).  Reductions are fixed-order
// shuffles and LDS trees, so results are bit-reproducible run to run.
//
// Sources (page title, section):
//   [QT-log] qwentts.cpp, commit log of src/pipeline-tts.h
//   [MC-opt] MiniCPM-o 4.5 single-GPU engine, docs/optimizations.md
#include "kernels.h"

#include <math.h>

namespace qtk {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t *p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

// float -> nearest bf16 (ties to even), kept in a float
__device__ __forceinline__ float bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return __uint_as_float((u | ((u & 0x7fffffu) ? 0x400000u : 0u)) & 0xffff0000u);
  u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint16_t bf16_bits(float f) { return (uint16_t)(__float_as_uint(bf16_rne(f)) >> 16); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float tab_at(const void *p, int bf16, size_t i) {
  return bf16 ? bf16_at((const uint16_t *)p, i) : ((const float *)p)[i];
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

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ int row_slot(const RowMap &m, int r) { return m.slot_base + r / m.rows_per_slot; }
__device__ __forceinline__ int row_pos(const RowMap &m, int r) {
  return m.pos_dev ? m.pos_dev[row_slot(m, r)] : m.pos_base + r % m.rows_per_slot;
}

// ------------------------------------------------------------------ GEMV
//
// One wave computes RW output rows; its 64 lanes split K into 16-byte chunks
// (8 bf16, 4 f32 or 16 int8 weights).  Activation rows are processed in
// groups of up to 8 held in registers, so each weight chunk is loaded once per
// group.

template <int WT> struct WT_;
template <> struct WT_<W_F32> { static constexpr int CH = 4; };
template <> struct WT_<W_BF16> { static constexpr int CH = 8; };
template <> struct WT_<W_Q8> { static constexpr int CH = 16; };

// dot of one 16-byte weight chunk with CH activations
template <int WT>
__device__ __forceinline__ float chunk_dot(const uint4 w, const float *xv, float scale) {
  if constexpr (WT == W_F32) {
    return __uint_as_float(w.x) * xv[0] + __uint_as_float(w.y) * xv[1] +
           __uint_as_float(w.z) * xv[2] + __uint_as_float(w.w) * xv[3];
  } else if constexpr (WT == W_BF16) {
    float s = bf16_lo(w.x) * xv[0];
    s += bf16_hi(w.x) * xv[1];
    s += bf16_lo(w.y) * xv[2];
    s += bf16_hi(w.y) * xv[3];
    s += bf16_lo(w.z) * xv[4];
    s += bf16_hi(w.z) * xv[5];
    s += bf16_lo(w.w) * xv[6];
    s += bf16_hi(w.w) * xv[7];
    return s;
  } else {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) s += (float)(int8_t)(ws[i] >> (8 * b)) * xv[4 * i + b];
    }
    return s * scale;
  }
}

template <int WT>
__device__ __forceinline__ const uint8_t *row_ptr(const Lin &L, int n, int K) {
  constexpr size_t esz = WT == W_F32 ? 4 : (WT == W_BF16 ? 2 : 1);
  return (const uint8_t *)L.w + (size_t)n * K * esz;
}

template <int WT, int EPI, int RW>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  constexpr int CH = WT_<WT>::CH;
  constexpr int NW = EPI == EPI_GATED ? 2 * RW : RW;  // weight rows per wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = a.K;
  const int nchunk = K / CH;
  const int row0 = (blockIdx.x * 4 + wave) * RW;

  // weight row pointers of this wave
  const uint8_t *wp[NW];
  const uint16_t *sp[NW];
  bool live[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int n = row0 + r;
    live[r] = n < a.N;
    const int nn = live[r] ? n : 0;
    if constexpr (EPI == EPI_GATED) {
      wp[2 * r] = row_ptr<WT>(a.seg[0], nn, K);
      wp[2 * r + 1] = row_ptr<WT>(a.up, nn, K);
      sp[2 * r] = a.seg[0].sc ? a.seg[0].sc + (size_t)nn * (K / 32) : nullptr;
      sp[2 * r + 1] = a.up.sc ? a.up.sc + (size_t)nn * (K / 32) : nullptr;
    } else {
      int s = 0, base = 0;
      while (s + 1 < a.nseg && nn >= a.seg_end[s]) { base = a.seg_end[s]; ++s; }
      wp[r] = row_ptr<WT>(a.seg[s], nn - base, K);
      sp[r] = a.seg[s].sc ? a.seg[s].sc + (size_t)(nn - base) * (K / 32) : nullptr;
    }
  }

  for (int m0 = 0; m0 < a.M; m0 += 8) {
    const int mg = min(8, a.M - m0);
    float rinv[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) rinv[m] = 1.f;
    if (a.gain) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mg) {
          const float *xr = a.x + (size_t)(m0 + m) * a.x_stride;
          float s = 0.f;
          for (int k = lane * 4; k < K; k += 256) {
            const float4 v = *(const float4 *)(xr + k);
            s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
          }
          s = wave_sum(s);
          rinv[m] = 1.0f / sqrtf(s / (float)K + a.eps);
        }
      }
      if (a.normed_out && blockIdx.x == 0) {
        // the only writer of normed_out: block 0, rows of this group
        for (int m = 0; m < mg; ++m) {
          const float *xr = a.x + (size_t)(m0 + m) * a.x_stride;
          float *dst = a.normed_out + (size_t)(m0 + m) * K;
          float rv = rinv[0];
#pragma unroll
          for (int mm = 1; mm < 8; ++mm) if (mm == m) rv = rinv[mm];
          for (int k = threadIdx.x; k < K; k += 256) dst[k] = xr[k] * rv * tab_at(a.gain, a.gain_bf16, k);
        }
      }
    }

    float acc[8][NW];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int r = 0; r < NW; ++r) acc[m][r] = 0.f;

    for (int c = lane; c < nchunk; c += 64) {
      const int k0 = c * CH;
      uint4 wv[NW];
      float scl[NW];
#pragma unroll
      for (int r = 0; r < NW; ++r) {
        wv[r] = *(const uint4 *)(wp[r] + (size_t)c * 16);
        scl[r] = 1.f;
        if constexpr (WT == W_Q8) scl[r] = f16_to_f32(sp[r][k0 / 32]);
      }
      float g[CH];
      if (a.gain) {
#pragma unroll
        for (int i = 0; i < CH; ++i) g[i] = tab_at(a.gain, a.gain_bf16, k0 + i);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mg) {
          const float *xr = a.x + (size_t)(m0 + m) * a.x_stride + k0;
          float xv[CH];
#pragma unroll
          for (int i = 0; i < CH; i += 4) {
            const float4 v = *(const float4 *)(xr + i);
            xv[i] = v.x; xv[i + 1] = v.y; xv[i + 2] = v.z; xv[i + 3] = v.w;
          }
          if (a.gain) {
#pragma unroll
            for (int i = 0; i < CH; ++i) xv[i] = xv[i] * rinv[m] * g[i];
          }
          if (a.act_bf16) {
#pragma unroll
            for (int i = 0; i < CH; ++i) xv[i] = bf16_rne(xv[i]);
          }
#pragma unroll
          for (int r = 0; r < NW; ++r) acc[m][r] += chunk_dot<WT>(wv[r], xv, scl[r]);
        }
      }
    }

#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m < mg) {
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          float v, u = 0.f;
          if constexpr (EPI == EPI_GATED) {
            v = wave_sum(acc[m][2 * r]);
            u = wave_sum(acc[m][2 * r + 1]);
          } else {
            v = wave_sum(acc[m][r]);
          }
          if (lane == 0 && live[r]) {
            const int n = row0 + r;
            float *yp = a.y + (size_t)(m0 + m) * a.y_stride + n;
            if constexpr (EPI == EPI_STORE) {
              *yp = v;
            } else if constexpr (EPI == EPI_RESID) {
              const float nv = *yp + v;
              *yp = nv;
              if (a.copy_out) a.copy_out[(size_t)(m0 + m) * a.copy_stride + n] = nv;
            } else {
              *yp = silu(v) * u;
            }
          }
        }
      }
    }
  }
}

template <int WT, int EPI>
static hipError_t gemv_rw(const GemvArgs &a, hipStream_t s) {
  // rows per wave: enough blocks to cover the CUs with a few waves each
  int rw = a.N >= 8192 ? 4 : (a.N >= 2048 ? 2 : 1);
  const int rows_per_block = 4 * rw;
  const dim3 grid((a.N + rows_per_block - 1) / rows_per_block);
  if (rw == 4) hipLaunchKernelGGL((gemv_kernel<WT, EPI, 4>), grid, dim3(256), 0, s, a);
  else if (rw == 2) hipLaunchKernelGGL((gemv_kernel<WT, EPI, 2>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((gemv_kernel<WT, EPI, 1>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int WT>
static hipError_t gemv_epi(int epi, const GemvArgs &a, hipStream_t s) {
  if (epi == EPI_STORE) return gemv_rw<WT, EPI_STORE>(a, s);
  if (epi == EPI_RESID) return gemv_rw<WT, EPI_RESID>(a, s);
  return gemv_rw<WT, EPI_GATED>(a, s);
}

hipError_t launch_gemv(int wtype, int epi, const GemvArgs &a, hipStream_t s) {
  if (wtype == W_F32) return gemv_epi<W_F32>(epi, a, s);
  if (wtype == W_BF16) return gemv_epi<W_BF16>(epi, a, s);
  return gemv_epi<W_Q8>(epi, a, s);
}

// ------------------------------------------------------------------ q/k norm + RoPE + set_rows
//
// One wave per (row, head).  Lane l owns the RoPE pair (i, i + hd/2) with
// i = l (hd = 128) or lanes 0..31 (hd = 64).  K and V rows are written to the
// ring at the row's position, read from device memory, so the step's graph
// does not depend on the position ([QT-log] set_rows entry; [MC-opt] core
// table, q/k norm + RoPE + v copy).

template <int HD, bool KVB>
__global__ __launch_bounds__(64) void qk_rope_kv_kernel(QkArgs a) {
  constexpr int HALF = HD / 2;
  const int r = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int slot = row_slot(a.rows, r), pos = row_pos(a.rows, r);
  const int qd = a.nq * HD, kd = a.nkv * HD;
  const float *row = a.qkv + (size_t)r * (qd + 2 * kd);
  const bool isq = h < a.nq;
  const int kh = h - a.nq;
  const float *src = isq ? row + h * HD : row + qd + kh * HD;
  const void *gain = isq ? a.q_gain : a.k_gain;
  const bool act = lane < HALF;
  float x0 = act ? src[lane] : 0.f, x1 = act ? src[lane + HALF] : 0.f;
  const float s = wave_sum(x0 * x0 + x1 * x1);
  const float rv = 1.0f / sqrtf(s / (float)HD + a.eps);
  if (!act) return;
  const float y0 = x0 * rv * tab_at(gain, a.gain_bf16, lane);
  const float y1 = x1 * rv * tab_at(gain, a.gain_bf16, lane + HALF);
  const float c = a.rope_cos[(size_t)pos * HALF + lane], sn = a.rope_sin[(size_t)pos * HALF + lane];
  const float o0 = y0 * c - y1 * sn;
  const float o1 = y1 * c + y0 * sn;
  if (isq) {
    float *dst = a.q_out + (size_t)r * qd + h * HD;
    dst[lane] = o0;
    dst[lane + HALF] = o1;
    return;
  }
  const size_t off = (size_t)slot * a.slot_stride + (size_t)kh * a.P * HD + (size_t)pos * HD;
  const float *vsrc = row + qd + kd + kh * HD;
  const float v0 = vsrc[lane], v1 = vsrc[lane + HALF];
  if constexpr (KVB) {
    uint16_t *kr = (uint16_t *)a.ring_layer + off;
    uint16_t *vr = kr + a.kv_stride;
    kr[lane] = bf16_bits(o0);
    kr[lane + HALF] = bf16_bits(o1);
    vr[lane] = bf16_bits(v0);
    vr[lane + HALF] = bf16_bits(v1);
  } else {
    float *kr = (float *)a.ring_layer + off;
    float *vr = kr + a.kv_stride;
    kr[lane] = o0;
    kr[lane + HALF] = o1;
    vr[lane] = v0;
    vr[lane + HALF] = v1;
  }
}

hipError_t launch_qk_rope_kv(int hd, int kv_bf16, const QkArgs &a, hipStream_t s) {
  const dim3 grid(a.M, a.nq + a.nkv);
  if (hd == 128) {
    if (kv_bf16) hipLaunchKernelGGL((qk_rope_kv_kernel<128, true>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((qk_rope_kv_kernel<128, false>), grid, dim3(64), 0, s, a);
  } else {
    if (kv_bf16) hipLaunchKernelGGL((qk_rope_kv_kernel<64, true>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((qk_rope_kv_kernel<64, false>), grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ attention
//
// Split-K decode attention.  Block (row, kv head, tile) covers positions
// [tile*T, tile*T + T) at fixed absolute boundaries for the GQA group of
// nq/nkv query heads.  Positions past the row's own (the padded tail of the
// window, [QT-log] persistent arena entry) are excluded by select and never
// read.  One tile: the block normalises and writes o; several: it writes
// (max, sum, acc) partials that the combine kernel merges in tile order.

template <int HD, int G, bool KVB>
__global__ __launch_bounds__(256) void attn_tile_kernel(AttnArgs a) {
  const int r = blockIdx.x, kh = blockIdx.y, t = blockIdx.z;
  const int slot = row_slot(a.rows, r), pos = row_pos(a.rows, r);
  const int j0 = t * a.tile;
  if (j0 > pos) return;
  const int jn = min(a.tile, pos + 1 - j0);
  const int ntiles = (pos + a.tile) / a.tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ float qs[G][HD];
  __shared__ float sc[G][256];
  __shared__ float red[G][4];
  __shared__ float stat[G][2];

  for (int i = tid; i < G * HD; i += 256)
    qs[i / HD][i % HD] = a.q[(size_t)r * a.nq * HD + (size_t)kh * G * HD + i];
  __syncthreads();

  const size_t head_off = (size_t)slot * a.slot_stride + (size_t)kh * a.P * HD;
  // scores: one thread per position
  if (tid < a.tile) {
    if (tid < jn) {
      float s[G];
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = 0.f;
      const size_t roff = head_off + (size_t)(j0 + tid) * HD;
      for (int d = 0; d < HD; d += 8) {
        float kv[8];
        if constexpr (KVB) {
          const uint4 w = *(const uint4 *)((const uint16_t *)a.ring_layer + roff + d);
          kv[0] = bf16_lo(w.x); kv[1] = bf16_hi(w.x); kv[2] = bf16_lo(w.y); kv[3] = bf16_hi(w.y);
          kv[4] = bf16_lo(w.z); kv[5] = bf16_hi(w.z); kv[6] = bf16_lo(w.w); kv[7] = bf16_hi(w.w);
        } else {
          const float4 v0 = *(const float4 *)((const float *)a.ring_layer + roff + d);
          const float4 v1 = *(const float4 *)((const float *)a.ring_layer + roff + d + 4);
          kv[0] = v0.x; kv[1] = v0.y; kv[2] = v0.z; kv[3] = v0.w;
          kv[4] = v1.x; kv[5] = v1.y; kv[6] = v1.z; kv[7] = v1.w;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int i = 0; i < 8; ++i) s[g] += qs[g][d + i] * kv[i];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g][tid] = s[g] * a.scale;
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g][tid] = -INFINITY;
    }
  }
  __syncthreads();

  // per query head: max, exp, sum (block tree in fixed order)
  for (int g = 0; g < G; ++g) {
    float v = (tid < a.tile) ? sc[g][tid] : -INFINITY;
    v = wave_max(v);
    if (lane == 0) red[g][wave] = v;
  }
  __syncthreads();
  if (tid < G) stat[tid][0] = fmaxf(fmaxf(red[tid][0], red[tid][1]), fmaxf(red[tid][2], red[tid][3]));
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    float e = 0.f;
    if (tid < jn) e = expf(sc[g][tid] - stat[g][0]);
    if (tid < a.tile) sc[g][tid] = e;
    e = wave_sum(e);
    if (lane == 0) red[g][wave] = e;
  }
  __syncthreads();
  if (tid < G) stat[tid][1] = (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]);
  __syncthreads();

  // P.V: thread (g, d)
  if (tid < G * HD) {
    const int g = tid / HD, d = tid % HD;
    float acc = 0.f;
    const size_t voff = head_off + a.kv_stride + (size_t)j0 * HD + d;
    for (int j = 0; j < jn; ++j) {
      const float v = KVB ? bf16_at((const uint16_t *)a.ring_layer, voff + (size_t)j * HD)
                          : ((const float *)a.ring_layer)[voff + (size_t)j * HD];
      acc += sc[g][j] * v;
    }
    const int h = kh * G + g;
    if (ntiles == 1) {
      a.o[(size_t)r * a.nq * HD + (size_t)h * HD + d] = acc / stat[g][1];
    } else {
      float *p = a.part + (((size_t)r * a.nq + h) * a.max_tiles + t) * (HD + 2);
      p[d] = acc;
      if (d == 0) {
        p[HD] = stat[g][0];
        p[HD + 1] = stat[g][1];
      }
    }
  }
}

template <int HD>
__global__ __launch_bounds__(HD) void attn_combine_kernel(AttnArgs a) {
  const int r = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int pos = row_pos(a.rows, r);
  const int ntiles = (pos + a.tile) / a.tile;
  if (ntiles == 1) return;
  const float *p = a.part + ((size_t)r * a.nq + h) * a.max_tiles * (HD + 2);
  float mx = -INFINITY;
  for (int t = 0; t < ntiles; ++t) mx = fmaxf(mx, p[(size_t)t * (HD + 2) + HD]);
  float L = 0.f, O = 0.f;
  for (int t = 0; t < ntiles; ++t) {
    const float *pt = p + (size_t)t * (HD + 2);
    const float w = expf(pt[HD] - mx);
    L += pt[HD + 1] * w;
    O += pt[d] * w;
  }
  a.o[(size_t)r * a.nq * HD + (size_t)h * HD + d] = O / L;
}

template <int HD, int G>
static void attn_tile_g(int kv_bf16, const AttnArgs &a, hipStream_t s) {
  const dim3 grid(a.M, a.nkv, a.max_tiles);
  if (kv_bf16) hipLaunchKernelGGL((attn_tile_kernel<HD, G, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((attn_tile_kernel<HD, G, false>), grid, dim3(256), 0, s, a);
}

template <int HD>
static void attn_tile_hd(int kv_bf16, const AttnArgs &a, hipStream_t s) {
  switch (a.nq / a.nkv) {
    case 1: attn_tile_g<HD, 1>(kv_bf16, a, s); break;
    case 2: attn_tile_g<HD, 2>(kv_bf16, a, s); break;
    default: attn_tile_g<HD, 4>(kv_bf16, a, s); break;  // host admits 1, 2, 4 (and 4*hd <= 256)
  }
}

hipError_t launch_attention(int hd, int kv_bf16, const AttnArgs &a, bool combine, hipStream_t s) {
  if (hd == 128) attn_tile_hd<128>(kv_bf16, a, s);
  else attn_tile_hd<64>(kv_bf16, a, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !combine) return e;
  const dim3 g2(a.M, a.nq);
  if (hd == 128) hipLaunchKernelGGL((attn_combine_kernel<128>), g2, dim3(128), 0, s, a);
  else hipLaunchKernelGGL((attn_combine_kernel<64>), g2, dim3(64), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ gather-sum
//
// Talker input: sum of the G code rows plus the overlay row, accumulated in
// f32 left to right ([QT-log] AR inputs on device entry).

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int r = blockIdx.x;
  const int i = blockIdx.y * 256 + threadIdx.x;
  const int f = a.ctl ? a.ctl[0] : 0;
  const int32_t *codes = a.codes ? a.codes + (size_t)f * a.frame_stride_codes + (size_t)r * a.codes_stride : nullptr;
  const int32_t text = a.text[(size_t)f * a.frame_stride_text + (size_t)r * a.text_stride];
  if (i < a.H) {
    float acc = 0.f;
    if (codes)
      for (int g = 0; g < a.G; ++g)
        acc += tab_at(a.code_emb, a.tab_bf16, ((size_t)g * a.Vc + codes[g]) * a.H + i);
    acc += tab_at(a.text_emb, a.tab_bf16, (size_t)text * a.H + i);
    a.x[(size_t)r * a.H + i] = acc;
    if (a.x0_dump) a.x0_dump[(size_t)r * a.H + i] = acc;
  }
  if (a.gather_dump && blockIdx.y == 0 && threadIdx.x <= a.G) {
    const int g = threadIdx.x;
    a.gather_dump[(size_t)r * (a.G + 1) + g] = g < a.G ? (codes ? codes[g] : -1) : text;
  }
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(gather_kernel, dim3(a.M, (a.H + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ predictor input
//
// Rows [bridge, E_0[c0]] of each stream's two-row predictor prefill
// ([QT-log] set_rows / bridge entry: the bridge is a leaf of the predictor
// prefill).  Also emits code 0 of the frame.

__global__ __launch_bounds__(256) void pred_input_kernel(PredInArgs a) {
  const int b = blockIdx.x;
  const int i = blockIdx.y * 256 + threadIdx.x;
  const int f = a.ctl[0] + a.k;
  const int force = a.ctl[1];
  int32_t *cin = a.cin + ((size_t)f * a.B + b) * a.G;
  int32_t *cout = a.cout + ((size_t)f * a.B + b) * a.G;
  const int c = force ? cin[0] : a.c0_state[b];
  if (i < a.H) {
    a.x[(size_t)(2 * b) * a.H + i] = a.bridge[(size_t)b * a.H + i];
    a.x[(size_t)(2 * b + 1) * a.H + i] = tab_at(a.code_emb, a.tab_bf16, (size_t)c * a.H + i);
  }
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    cout[0] = a.c0_state[b];
    if (!force) cin[0] = a.c0_state[b];
  }
}

hipError_t launch_pred_input(const PredInArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(pred_input_kernel, dim3(a.B, (a.H + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ argmax
//
// Greedy pick on device, lowest index on ties ([QT-tests] fused codec mode
// entry: in-graph sampler).  Predictor heads also gather the next micro-step's
// input row; the talker head advances the slot's position.

__global__ __launch_bounds__(256) void argmax_kernel(ArgmaxArgs a) {
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *lg = a.logits + (size_t)r * a.Vc;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = tid; i < a.Vc; i += 256) {
    const float v = lg[i];
    if (v > best) { best = v; bi = i; }   // increasing i: first max kept
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int code;
  if (lane == 0) { sv[wave] = best; si[wave] = bi; }
  __syncthreads();
  if (tid == 0) {
    float bv = sv[0];
    int b = si[0];
    for (int w = 1; w < 4; ++w)
      if (sv[w] > bv || (sv[w] == bv && si[w] < b)) { bv = sv[w]; b = si[w]; }
    if (b == 0x7fffffff) b = 0;  // all NaN: never expected
    int c = b;
    if (a.mode == AM_PRED) {
      const int f = a.ctl[0] + a.k;
      const size_t base = ((size_t)f * a.B + r) * a.G + a.j + 1;
      a.cout[base] = b;
      if (a.ctl[1]) c = a.cin[base];
      else a.cin[base] = b;
    } else if (a.mode == AM_TALKER) {
      a.c0_state[r] = b;
      if (a.tpos_dump) a.tpos_dump[r] = a.pos[r];
      a.pos[r] = a.pos[r] + 1;
    } else {
      a.c0_state[a.slot] = b;
    }
    code = c;
  }
  if (a.mode == AM_PRED && a.x_next && a.j + 2 < a.G) {
    __syncthreads();
    const int c = code;
    const size_t base = ((size_t)(a.j + 1) * a.Vc + c) * a.H;
    for (int i = tid; i < a.H; i += 256) a.x_next[(size_t)r * a.H + i] = tab_at(a.code_emb, a.tab_bf16, base + i);
  }
}

hipError_t launch_argmax(const ArgmaxArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(argmax_kernel, dim3(a.M), dim3(256), 0, s, a);
  return hipGetLastError();
}

__global__ void advance_kernel(int32_t *ctl, int32_t K) {
  if (threadIdx.x == 0) ctl[0] = ctl[0] + K;
}

hipError_t launch_advance(int32_t *ctl, int32_t K, hipStream_t s) {
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, s, ctl, K);
  return hipGetLastError();
}

}  // namespace qtk
