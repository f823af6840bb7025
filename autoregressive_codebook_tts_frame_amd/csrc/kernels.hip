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
#include "sampler.h"

#include <math.h>
#include <type_traits>

namespace qtk {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t *p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

// float -> nearest bf16 (ties to even), kept in a float
__device__ __forceinline__ float bf16_rne(float f) {
  return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f) << 16);
}
__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

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

// PFM: the rows are a prompt chunk's (m.pf set), a separate instantiation of
// each kernel, so the decode steps' rows carry no descriptor reads or checks
template <bool PFM>
__device__ __forceinline__ int row_slot(const RowMap &m, int r) {
  if constexpr (PFM) return m.pf[PF_SLOT + r / m.rows_per_slot];
  return m.slot_base + r / m.rows_per_slot;
}
template <bool PFM>
__device__ __forceinline__ int row_pos(const RowMap &m, int r) {
  if constexpr (PFM) return m.pf[PF_R0] + r % m.rows_per_slot;
  return m.pos_dev ? m.pos_dev[row_slot<false>(m, r)] : m.pos_base + r % m.rows_per_slot;
}
// false for a prompt chunk's padding rows (their stream's prompt has ended)
template <bool PFM>
__device__ __forceinline__ bool row_valid(const RowMap &m, int r) {
  if constexpr (PFM) return r % m.rows_per_slot < m.pf[PF_LEN + r / m.rows_per_slot];
  return true;
}
// Element offset of (slot, position) inside one (layer, K|V) block of the
// ring, head kh: the dense ring [slot][head][P][hd], or the paged pool
// [head][rows][hd] with the position's row from the page table (page size 1:
// each position's row is placed independently, the table carried as data).
template <int HD>
__device__ __forceinline__ size_t ring_off(const int32_t *ptab, int64_t slot_stride, int P, int rows_per_head,
                                           int slot, int kh, int pos) {
  if (ptab) return ((size_t)kh * rows_per_head + (size_t)ptab[(size_t)slot * P + pos]) * HD;
  return (size_t)slot * slot_stride + ((size_t)kh * P + pos) * HD;
}

// ------------------------------------------------------------------ GEMV
//
// One wave computes RW output rows; its 64 lanes split K into 16-byte chunks
// (8 bf16, 4 f32, 16 int8 or 32 4-bit weights: half a q8 block, one q4
// block).  Activation rows are processed in groups of up to 8 held in
// registers, so each weight chunk is loaded once per group.

template <int WT> struct WT_;
template <> struct WT_<W_F32> { static constexpr int CH = 4; };
template <> struct WT_<W_BF16> { static constexpr int CH = 8; };
template <> struct WT_<W_Q8> { static constexpr int CH = 16; };
template <> struct WT_<W_Q4> { static constexpr int CH = 32; };

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
  } else if constexpr (WT == W_Q8) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) s += (float)(int8_t)(ws[i] >> (8 * b)) * xv[4 * i + b];
    }
    return s * scale;
  } else {
    // nibble b of word i is weight 8 i + b
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int b = 0; b < 8; ++b) s += (float)((int)((ws[i] >> (4 * b)) & 15u) - 8) * xv[8 * i + b];
    }
    return s * scale;
  }
}

// bytes of one weight row of K weights (block scales are stored apart)
template <int WT>
__device__ __forceinline__ size_t row_bytes(int K) {
  return WT == W_F32 ? (size_t)K * 4 : WT == W_BF16 ? (size_t)K * 2 : WT == W_Q8 ? (size_t)K : (size_t)K / 2;
}

template <int WT>
__device__ __forceinline__ const uint8_t *row_ptr(const Lin &L, int n, int K) {
  return (const uint8_t *)L.w + (size_t)n * row_bytes<WT>(K);
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
        if constexpr (w_blocked(WT)) scl[r] = f16_to_f32(sp[r][k0 / 32]);
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
  if (wtype == W_Q8) return gemv_epi<W_Q8>(epi, a, s);
  if (wtype == W_Q4) return gemv_epi<W_Q4>(epi, a, s);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ q/k norm + RoPE + set_rows
//
// One wave per (row, head).  Lane l owns the RoPE pair (i, i + hd/2) with
// i = l (hd = 128) or lanes 0..31 (hd = 64).  K and V rows are written to the
// ring at the row's position, read from device memory, so the step's graph
// does not depend on the position ([QT-log] set_rows entry; [MC-opt] core
// table, q/k norm + RoPE + v copy).

// Per-head RMSNorm then NeoX RoPE of one head vector, one wave per vector:
// lane i < HD/2 holds the pair (x0, x1) = (x_i, x_{i+HD/2}) (the other lanes
// hold zeros and take part in the norm's sum only), its gains g0, g1 and the
// position's cos / sin, and gets the rotated pair in o0, o1.  Shared by the
// separate kernel and the fused attention prologue, so both round alike.
template <int HD>
__device__ __forceinline__ void qk_norm_rope(float x0, float x1, float g0, float g1, float c, float sn, float eps,
                                             float &o0, float &o1) {
  const float s = wave_sum(x0 * x0 + x1 * x1);
  const float rv = 1.0f / sqrtf(s / (float)HD + eps);
  const float y0 = x0 * rv * g0;
  const float y1 = x1 * rv * g1;
  o0 = y0 * c - y1 * sn;
  o1 = y1 * c + y0 * sn;
}

template <int HD, bool KVB, bool PFM>
__global__ __launch_bounds__(64) void qk_rope_kv_kernel(QkArgs a) {
  constexpr int HALF = HD / 2;
  const int r = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  if (!row_valid<PFM>(a.rows, r)) return;  // padding: nothing reaches the ring
  const int slot = row_slot<PFM>(a.rows, r), pos = row_pos<PFM>(a.rows, r);
  const int qd = a.nq * HD, kd = a.nkv * HD;
  const float *row = a.qkv + (size_t)r * (qd + 2 * kd);
  const bool isq = h < a.nq;
  const int kh = h - a.nq;
  const float *src = isq ? row + h * HD : row + qd + kh * HD;
  const void *gain = isq ? a.q_gain : a.k_gain;
  const bool act = lane < HALF;
  const float x0 = act ? src[lane] : 0.f, x1 = act ? src[lane + HALF] : 0.f;
  const int ln = act ? lane : 0;  // idle lanes read pair 0 (in bounds) and discard it
  float o0, o1;
  qk_norm_rope<HD>(x0, x1, tab_at(gain, a.gain_bf16, ln), tab_at(gain, a.gain_bf16, ln + HALF),
                   a.rope_cos[(size_t)pos * HALF + ln], a.rope_sin[(size_t)pos * HALF + ln], a.eps, o0, o1);
  if (!act) return;
  if (isq) {
    float *dst = a.q_out + (size_t)r * qd + h * HD;
    dst[lane] = o0;
    dst[lane + HALF] = o1;
    return;
  }
  const size_t off = ring_off<HD>(a.ptab, a.slot_stride, a.P, a.rows_per_head, slot, kh, pos);
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
  const bool pf = a.rows.pf != nullptr;
  if (hd == 128) {
    if (kv_bf16) {
      if (pf) hipLaunchKernelGGL((qk_rope_kv_kernel<128, true, true>), grid, dim3(64), 0, s, a);
      else hipLaunchKernelGGL((qk_rope_kv_kernel<128, true, false>), grid, dim3(64), 0, s, a);
    } else {
      if (pf) hipLaunchKernelGGL((qk_rope_kv_kernel<128, false, true>), grid, dim3(64), 0, s, a);
      else hipLaunchKernelGGL((qk_rope_kv_kernel<128, false, false>), grid, dim3(64), 0, s, a);
    }
  } else {
    if (kv_bf16) {
      if (pf) hipLaunchKernelGGL((qk_rope_kv_kernel<64, true, true>), grid, dim3(64), 0, s, a);
      else hipLaunchKernelGGL((qk_rope_kv_kernel<64, true, false>), grid, dim3(64), 0, s, a);
    } else {
      if (pf) hipLaunchKernelGGL((qk_rope_kv_kernel<64, false, true>), grid, dim3(64), 0, s, a);
      else hipLaunchKernelGGL((qk_rope_kv_kernel<64, false, false>), grid, dim3(64), 0, s, a);
    }
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

// Row sums over groups of L lanes (L = 8, 16 or 32); every lane of a group
// gets its group's sum.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <>
__device__ __forceinline__ float group_sum<16>(float v) {  // one DPP row
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, true));
  return v;
}

// 16-byte K/V chunk -> floats
template <bool KVB>
__device__ __forceinline__ void kv_unpack(uint4 w, float *v) {
  if constexpr (KVB) {
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else {
    v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y); v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
  }
}

// Lanes work in groups of CPR = one K/V row (16-byte chunk each): a row is one
// coalesced read, PG = 256 / CPR rows per pass, and every chunk a thread needs
// is requested before it is used.
// PAGED: the tile's rows come through the page table (a separate
// instantiation, so the dense ring's address arithmetic stays as it is).
template <int HD, int G, bool KVB, bool FUSED, bool PAGED, bool PFM>
__global__ __launch_bounds__(256) void attn_tile_kernel(AttnArgs a) {
  constexpr int ESZ = KVB ? 2 : 4;
  constexpr int DPC = 16 / ESZ;   // values per chunk
  constexpr int CPR = HD / DPC;   // chunks per row
  constexpr int PG = 256 / CPR;   // rows per pass
  constexpr int NP = 256 / PG;    // passes over a full tile
  const int r = blockIdx.x, kh = blockIdx.y, t = blockIdx.z;
  if (!row_valid<PFM>(a.rows, r)) return;  // padding rows attend to nothing
  const int slot = row_slot<PFM>(a.rows, r), pos = row_pos<PFM>(a.rows, r);
  const int j0 = t * a.tile;
  if (j0 > pos) return;
  const int jn = min(a.tile, pos + 1 - j0);
  const int ntiles = (pos + a.tile) / a.tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pg = tid / CPR, cc = tid % CPR;

  __shared__ float sc[G][256];
  __shared__ float stat[G][2];
  __shared__ float red[4][G][HD];
  __shared__ float qs[FUSED ? G : 1][HD];                                       // rotated queries
  __shared__ __attribute__((aligned(16))) uint32_t nrow[FUSED ? 2 : 1][2][HD * ESZ / 4];  // new K, V rows

  // Fused prologue (decode steps: one or two rows per slot).  Items, one wave
  // each: the G query heads of row r, then the K rows of head kh at the
  // slot's new positions that fall in this tile (a slot's second row also
  // attends to its first row's position).  Their inputs are requested first,
  // then the ring rows, so the prologue waits only for its own loads.
  constexpr int HALF = HD / 2;
  const int qd = a.nq * HD, kd = a.nkv * HD;
  int rs0 = r, p0 = pos, p1 = pos;
  bool need0 = false, need1 = false;
  constexpr int NS = (G + 2 + 3) / 4;  // prologue items per wave
  float fx0[NS], fx1[NS], fg0[NS], fg1[NS], fc[NS], fs[NS], fv0[NS], fv1[NS];
  if constexpr (FUSED) {
    const int rps = a.rows.rows_per_slot;
    rs0 = r - r % rps;
    p0 = row_pos<PFM>(a.rows, rs0);
    p1 = rps > 1 ? row_pos<PFM>(a.rows, rs0 + 1) : pos;
    need0 = p0 >= j0 && p0 - j0 < jn;  // inside this tile, at or before pos
    need1 = rps > 1 && p1 >= j0 && p1 - j0 < jn;
    const int ln = lane & (HALF - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int it = wave + 4 * s, i = it - G;
      const bool isq = it < G, isk = (i == 0 && need0) || (i == 1 && need1);
      const int rr = isk ? rs0 + i : r, pp = isk ? (i ? p1 : p0) : pos;
      const float *row = a.qkv + (size_t)rr * (qd + 2 * kd);
      const float *src = isk ? row + qd + kh * HD : row + (kh * G + (isq ? it : 0)) * HD;
      const void *gain = isk ? a.k_gain : a.q_gain;
      fx0[s] = src[ln];
      fx1[s] = src[ln + HALF];
      fg0[s] = tab_at(gain, a.gain_bf16, ln);
      fg1[s] = tab_at(gain, a.gain_bf16, ln + HALF);
      fc[s] = a.rope_cos[(size_t)pp * HALF + ln];
      fs[s] = a.rope_sin[(size_t)pp * HALF + ln];
      fv0[s] = row[qd + kd + kh * HD + ln];
      fv1[s] = row[qd + kd + kh * HD + ln + HALF];
    }
  }

  // This thread's q chunks (unfused), then the tile's K rows, then its V
  // rows, all requested before the first use of any of them (in that order,
  // so each use waits only for what it needs).  The loads are unconditional:
  // rows past the context read the tile's row 0 and are never used (a load
  // skipped by a branch would make the compiler wait for every load at the
  // join).
  float qr[G][DPC];
  if constexpr (!FUSED) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float *qp = a.q + (size_t)r * a.nq * HD + (size_t)(kh * G + g) * HD + cc * DPC;
#pragma unroll
      for (int e = 0; e < DPC; e += 4) {
        const float4 v = *(const float4 *)(qp + e);
        qr[g][e] = v.x; qr[g][e + 1] = v.y; qr[g][e + 2] = v.z; qr[g][e + 3] = v.w;
      }
    }
  }
  // this thread's rows j = p * PG + pg of the tile (position j0 + j): K at
  // ring + roff, V one K|V block further (dense: consecutive positions;
  // paged: each row from the page table, all table entries read first)
  const size_t head_off = (size_t)slot * a.slot_stride + (size_t)kh * a.P * HD;
  const uint8_t *kbase = (const uint8_t *)a.ring_layer + (head_off + (size_t)j0 * HD) * ESZ;
  const uint8_t *vbase = (const uint8_t *)a.ring_layer + (head_off + a.kv_stride + (size_t)j0 * HD) * ESZ;
  size_t roff[PAGED ? NP : 1];  // paged: byte offset of each row's K chunk (V one K|V block further)
  if constexpr (PAGED) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int j = p * PG + pg;
      roff[p] = ring_off<HD>(a.ptab, 0, a.P, a.rows_per_head, slot, kh, j0 + (j < jn ? j : 0)) * ESZ + cc * 16;
    }
  }
  auto krow = [&](int p) -> const uint4 * {
    const int j = p * PG + pg;
    if constexpr (PAGED) return (const uint4 *)((const uint8_t *)a.ring_layer + roff[p]);
    return (const uint4 *)(kbase + (size_t)(j < jn ? j : 0) * HD * ESZ + cc * 16);
  };
  auto vrow = [&](int p) -> const uint4 * {
    const int j = p * PG + pg;
    if constexpr (PAGED) return (const uint4 *)((const uint8_t *)a.ring_layer + roff[p] + (size_t)a.kv_stride * ESZ);
    return (const uint4 *)(vbase + (size_t)(j < jn ? j : 0) * HD * ESZ + cc * 16);
  };
  uint4 kc[NP], vc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) kc[p] = *krow(p);

  if constexpr (FUSED) {
    const bool act = lane < HALF;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int it = wave + 4 * s, i = it - G;
      const bool isq = it < G, isk = (i == 0 && need0) || (i == 1 && need1);
      if (!isq && !isk) continue;  // wave-uniform
      float o0, o1;
      qk_norm_rope<HD>(act ? fx0[s] : 0.f, act ? fx1[s] : 0.f, fg0[s], fg1[s], fc[s], fs[s], a.eps, o0, o1);
      if (!act) continue;
      if (isq) {
        qs[it][lane] = o0;
        qs[it][lane + HALF] = o1;
        continue;
      }
      const float v0 = fv0[s], v1 = fv1[s];
      // the row in its storage format, as the ring holds it
      if constexpr (KVB) {
        uint16_t *kr = (uint16_t *)nrow[i][0], *vr = (uint16_t *)nrow[i][1];
        kr[lane] = bf16_bits(o0); kr[lane + HALF] = bf16_bits(o1);
        vr[lane] = bf16_bits(v0); vr[lane + HALF] = bf16_bits(v1);
      } else {
        float *kr = (float *)nrow[i][0], *vr = (float *)nrow[i][1];
        kr[lane] = o0; kr[lane + HALF] = o1;
        vr[lane] = v0; vr[lane + HALF] = v1;
      }
      if (rs0 + i == r) {
        // set_rows: the row's own workgroup (its last tile) writes its K/V row
        const size_t off = head_off + (size_t)pos * HD;  // (the fused prologue serves the dense predictor cache)
        if constexpr (KVB) {
          uint16_t *kr = (uint16_t *)a.ring_layer + off, *vr = kr + a.kv_stride;
          kr[lane] = bf16_bits(o0); kr[lane + HALF] = bf16_bits(o1);
          vr[lane] = bf16_bits(v0); vr[lane + HALF] = bf16_bits(v1);
        } else {
          float *kr = (float *)a.ring_layer + off, *vr = kr + a.kv_stride;
          kr[lane] = o0; kr[lane + HALF] = o1;
          vr[lane] = v0; vr[lane + HALF] = v1;
        }
      }
    }
    __syncthreads();  // K/V loads stay in flight: the barrier waits for LDS operations only
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < DPC; ++e) qr[g][e] = qs[g][cc * DPC + e];
  }
  // V rows, requested after the prologue (whose inputs are dead by now)
#pragma unroll
  for (int p = 0; p < NP; ++p) vc[p] = *vrow(p);

  // Rows of the step's new positions come from the workgroup, not from the
  // ring: the loops below skip them, and they are added after each loop.  A
  // new position is the last valid row of its lane group (at most two
  // consecutive new positions, at least 8 rows per pass), so the sums keep
  // their order.
  auto is_new = [&](int j) { return FUSED && ((need0 && j0 + j == p0) || (need1 && j0 + j == p1)); };

  // scores
  {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (p * PG >= jn) break;
      const int j = p * PG + pg;
      float kf[8];
      kv_unpack<KVB>(kc[p], kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < DPC; ++e) d += qr[g][e] * kf[e];
        d = group_sum<CPR>(d);
        if (cc == 0 && j < jn && !is_new(j)) sc[g][j] = d * a.scale;
      }
    }
    if constexpr (FUSED)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int jl = (i ? p1 : p0) - j0;
        if (!(i ? need1 : need0) || pg != jl % PG) continue;  // uniform over the lane group
        float kf[8];
        kv_unpack<KVB>(((const uint4 *)nrow[i][0])[cc], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < DPC; ++e) d += qr[g][e] * kf[e];
          d = group_sum<CPR>(d);
          if (cc == 0) sc[g][jl] = d * a.scale;
        }
      }
  }
  __syncthreads();
  // softmax statistics: one wave per query head
  for (int g = wave; g < G; g += 4) {
    float mx = -INFINITY;
    for (int j = lane; j < jn; j += 64) mx = fmaxf(mx, sc[g][j]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int j = lane; j < jn; j += 64) {
      const float e = expf(sc[g][j] - mx);
      sc[g][j] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) { stat[g][0] = mx; stat[g][1] = sum; }
  }
  __syncthreads();
  // P.V: lanes (pg, chunk cc) accumulate their rows
  {
    float acc[G][DPC];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < DPC; ++e) acc[g][e] = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (p * PG >= jn) break;
      const int j = p * PG + pg;
      if (j < jn && !is_new(j)) {
        float vf[8];
        kv_unpack<KVB>(vc[p], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float e = sc[g][j];
#pragma unroll
          for (int d = 0; d < DPC; ++d) acc[g][d] += e * vf[d];
        }
      }
    }
    if constexpr (FUSED)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int jl = (i ? p1 : p0) - j0;
        if (!(i ? need1 : need0) || pg != jl % PG) continue;
        float vf[8];
        kv_unpack<KVB>(((const uint4 *)nrow[i][1])[cc], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float e = sc[g][jl];
#pragma unroll
          for (int d = 0; d < DPC; ++d) acc[g][d] += e * vf[d];
        }
      }
    // row groups inside the wave (lanes cc, cc + CPR, ...), then across waves
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int d = 0; d < DPC; ++d)
#pragma unroll
        for (int o = CPR; o < 64; o <<= 1) acc[g][d] += __shfl_xor(acc[g][d], o, 64);
    if (lane < CPR)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int d = 0; d < DPC; ++d) red[wave][g][cc * DPC + d] = acc[g][d];
  }
  __syncthreads();
  for (int i = tid; i < G * HD; i += 256) {
    const int g = i / HD, d = i % HD;
    const float o = (red[0][g][d] + red[1][g][d]) + (red[2][g][d] + red[3][g][d]);
    const int h = kh * G + g;
    if (ntiles == 1) {
      a.o[(size_t)r * a.nq * HD + (size_t)h * HD + d] = o / stat[g][1];
    } else {
      float *p = a.part + (((size_t)r * a.nq + h) * a.max_tiles + t) * (HD + 2);
      p[d] = o;
      if (d == 0) {
        p[HD] = stat[g][0];
        p[HD + 1] = stat[g][1];
      }
    }
  }
}

template <int HD, bool PFM>
__global__ __launch_bounds__(HD) void attn_combine_kernel(AttnArgs a) {
  const int r = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  if (!row_valid<PFM>(a.rows, r)) return;
  const int pos = row_pos<PFM>(a.rows, r);
  const int ntiles = (pos + a.tile) / a.tile;
  if (ntiles == 1) return;
  const float *p = a.part + ((size_t)r * a.nq + h) * a.max_tiles * (HD + 2);
  // Tiles in groups of 16 with every load of a group in flight at once.  Up
  // to 16 tiles (2,048 positions) this is the plain two-pass merge: the
  // group's maximum, then its weighted sums in tile order; later groups are
  // merged online (the running sums rescaled to the new maximum).
  constexpr int TG = 16;
  float mx = -INFINITY, L = 0.f, O = 0.f;
  for (int t0 = 0; t0 < ntiles; t0 += TG) {
    float mv[TG], lv[TG], ov[TG];
#pragma unroll
    for (int u = 0; u < TG; ++u) {
      const float *pt = p + (size_t)min(t0 + u, ntiles - 1) * (HD + 2);
      mv[u] = pt[HD];
      lv[u] = pt[HD + 1];
      ov[u] = pt[d];
    }
    float cm = mx;
#pragma unroll
    for (int u = 0; u < TG; ++u)
      if (t0 + u < ntiles) cm = fmaxf(cm, mv[u]);
    if (t0 > 0) {
      const float sc = expf(mx - cm);
      L *= sc;
      O *= sc;
    }
#pragma unroll
    for (int u = 0; u < TG; ++u)
      if (t0 + u < ntiles) {
        const float w = expf(mv[u] - cm);
        L += lv[u] * w;
        O += ov[u] * w;
      }
    mx = cm;
  }
  a.o[(size_t)r * a.nq * HD + (size_t)h * HD + d] = O / L;
}

template <int HD, int G>
static void attn_tile_g(int kv_bf16, const AttnArgs &a, hipStream_t s) {
  const dim3 grid(a.M, a.nkv, a.grid_tiles > 0 ? a.grid_tiles : a.max_tiles);
  if (a.qkv) {  // (the predictor's dense cache: never paged, never a prompt chunk)
    if (kv_bf16) hipLaunchKernelGGL((attn_tile_kernel<HD, G, true, true, false, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_tile_kernel<HD, G, false, true, false, false>), grid, dim3(256), 0, s, a);
  } else if (a.rows.pf) {  // prompt chunks of the shapes the MFMA kernel does not take
    if (a.ptab) {
      if (kv_bf16) hipLaunchKernelGGL((attn_tile_kernel<HD, G, true, false, true, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((attn_tile_kernel<HD, G, false, false, true, true>), grid, dim3(256), 0, s, a);
    } else {
      if (kv_bf16) hipLaunchKernelGGL((attn_tile_kernel<HD, G, true, false, false, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((attn_tile_kernel<HD, G, false, false, false, true>), grid, dim3(256), 0, s, a);
    }
  } else if (a.ptab) {
    if (kv_bf16) hipLaunchKernelGGL((attn_tile_kernel<HD, G, true, false, true, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_tile_kernel<HD, G, false, false, true, false>), grid, dim3(256), 0, s, a);
  } else {
    if (kv_bf16) hipLaunchKernelGGL((attn_tile_kernel<HD, G, true, false, false, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_tile_kernel<HD, G, false, false, false, false>), grid, dim3(256), 0, s, a);
  }
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
  if (a.qkv && a.ptab) return hipErrorInvalidValue;  // the fused prologue writes the dense cache only
  if (hd == 128) attn_tile_hd<128>(kv_bf16, a, s);
  else attn_tile_hd<64>(kv_bf16, a, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !combine) return e;
  const dim3 g2(a.M, a.nq);
  if (a.rows.pf) {
    if (hd == 128) hipLaunchKernelGGL((attn_combine_kernel<128, true>), g2, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((attn_combine_kernel<64, true>), g2, dim3(64), 0, s, a);
  } else {
    if (hd == 128) hipLaunchKernelGGL((attn_combine_kernel<128, false>), g2, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((attn_combine_kernel<64, false>), g2, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ prompt-chunk attention (MFMA)
//
// Causal attention of a prompt chunk's rows ([QT-log] per-layer K/V ring
// entry: a prompt row attends to every earlier position and its own).  The
// decode tile kernel gives each query row a workgroup, which for a long
// prompt reads every K/V tile once per row; here a workgroup takes 16 query
// positions of one stream and the G query heads of one KV head, and reads
// each K/V row of their range once.  The products run on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) with f32 accumulation: the K/V rows are bf16
// already, and each f32 query and probability enters as two bf16 terms, hi =
// bf16(v) and lo = bf16(v - hi) (v - hi is exact), so a product carries 16
// bits of the f32 operand where one bf16 term would carry 8.
// Waves (g, part): query head kh*G + g over the 64-position key blocks kb
// with kb % NPART == part, each with its own online softmax; the parts are
// merged at the end in a fixed order, so every row's result depends on its
// position only (chunks of any size give the same bits).  A block's K rows go
// straight to registers and its V rows through LDS (d-major), both requested
// before the block's barrier.
//   S^T = K Q^T per 16 keys: A = K (lane: key l%16, d = 32 st + 8 (l/16) ..
//   + 8 at step st), B = Q^T (the same d, query l%16); D[r] = score of key
//   4 (l/16) + r and query l%16.  O = P V per 32 keys (sub-blocks 2j, 2j+1):
//   A = P (query l%16; its 8 k slots are the lane's own scores, keys
//   4 (l/16) + r of both sub-blocks), B = V (the same keys, d = 16 db + l%16)
//   from a d-major copy of the block in LDS; D[r] = O[query 4 (l/16) + r][d
//   16 db + l%16].
constexpr int PKB = 64;  // key positions per block
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
// v as bf16 hi + lo terms (hi = nearest bf16, lo = nearest bf16 of the exact v - hi)
__device__ __forceinline__ void split_bf16(const f32x8_t v, bf16x8_t &hi, bf16x8_t &lo) {
  hi = __builtin_convertvector(v, bf16x8_t);
  lo = __builtin_convertvector(v - __builtin_convertvector(hi, f32x8_t), bf16x8_t);
}

constexpr int PNPART = 4;  // key-block partitions per workgroup (G = 1: 4 waves, G = 2: 8)

template <int G>
__global__ __launch_bounds__(64 * G * PNPART) void attn_prompt_kernel(AttnArgs a) {
  constexpr int HD = 128;
  constexpr int NPART = PNPART;
  constexpr int DPT = HD / G;  // d values each staging thread copies
  __shared__ __attribute__((aligned(16))) uint16_t vt[NPART][HD][PKB + 4];  // V^T of each part's block (+4: banks)
  __shared__ f32x4_t mo[NPART - 1][G][8][64];                              // parts 1..'s O
  __shared__ float ml[NPART - 1][G][2][16];                                // parts 1..'s (m, l)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = wave % G, part = wave / G;
  const int kh = blockIdx.y;
  const int t = a.rows.rows_per_slot, nqb = (t + 15) / 16;
  const int si = blockIdx.x / nqb, qoff = (blockIdx.x % nqb) * 16;
  const int32_t *pf = a.rows.pf;
  const int len = pf[PF_LEN + si];
  if (qoff >= len) return;  // padding only (the whole workgroup)
  const int nval = min(16, len - qoff);
  const int slot = pf[PF_SLOT + si];
  const int p0 = pf[PF_R0] + qoff, pmax = p0 + nval - 1;
  const int nkb = pmax / PKB + 1, niter = (nkb + NPART - 1) / NPART;
  const int row0 = si * t + qoff;  // chunk row of query 0
  const int h = kh * G + g;
  const int ql = lane & 15, kq = lane >> 4;
  const int qpos = p0 + ql;
  const uint16_t *ring = (const uint16_t *)a.ring_layer;

  bf16x8_t qhi[4], qlo[4];  // this lane's query values, d = 32 st + 8 kq .. + 8
  {
    const float *qp = a.q + (size_t)(row0 + min(ql, nval - 1)) * a.nq * HD + (size_t)h * HD + 8 * kq;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float4 v0 = *(const float4 *)(qp + 32 * st), v1 = *(const float4 *)(qp + 32 * st + 4);
      split_bf16((f32x8_t){v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w}, qhi[st], qlo[st]);
    }
  }
  const int ptid = g * 64 + lane;  // staging thread within the part
  const int vk = ptid & (PKB - 1), vd0 = (ptid / PKB) * DPT;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t O[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) O[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < niter; ++it) {
    const int kb = NPART * it + part;
    const bool active = kb < nkb;  // wave-uniform
    // the block's K rows (to registers) and V rows, requested together; rows
    // past the last query position read that position's row (never used)
    uint4 kw[4][4];  // [sub-block][st]: key l%16 of the sub-block, d = 32 st + 8 kq .. + 8
    if (active) {
      const int pos = min(kb * PKB + vk, pmax);
      const uint16_t *vr = ring + ring_off<HD>(a.ptab, a.slot_stride, a.P, a.rows_per_head, slot, kh, pos) +
                           a.kv_stride + vd0;
      uint4 w[DPT / 8];
#pragma unroll
      for (int c = 0; c < DPT / 8; ++c) w[c] = *(const uint4 *)(vr + 8 * c);
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        const int kpos = min(kb * PKB + sb * 16 + ql, pmax);
        const uint16_t *kr = ring + ring_off<HD>(a.ptab, a.slot_stride, a.P, a.rows_per_head, slot, kh, kpos) + 8 * kq;
#pragma unroll
        for (int st = 0; st < 4; ++st) kw[sb][st] = *(const uint4 *)(kr + 32 * st);
      }
      // V^T of block kb
#pragma unroll
      for (int c = 0; c < DPT / 8; ++c) {
        const uint32_t ww[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt[part][vd0 + 8 * c + 2 * e][vk] = (uint16_t)(ww[e] & 0xffffu);
          vt[part][vd0 + 8 * c + 2 * e + 1][vk] = (uint16_t)(ww[e] >> 16);
        }
      }
    }
    __syncthreads();
    if (active) {
      // scores of the block's 4 sub-blocks of 16 keys
      f32x4_t s[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, kw[sb][st]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qhi[st], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qlo[st], acc, 0, 0, 0);
        }
        s[sb] = acc;
      }
      // online softmax: scale, causal mask, the block's maximum per query
      float mb = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb * PKB + sb * 16 + 4 * kq + r;
          const float v = key > qpos ? -INFINITY : s[sb][r] * a.scale;
          s[sb][r] = v;
          mb = fmaxf(mb, v);
        }
      mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
      const float m_new = fmaxf(m_run, mb);
      const float corr = m_new == -INFINITY ? 1.f : expf(m_run - m_new);
      float ps = 0.f;
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = s[sb][r] == -INFINITY ? 0.f : expf(s[sb][r] - m_new);
          s[sb][r] = p;
          ps += p;
        }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_run = l_run * corr + ps;
      m_run = m_new;
      // O rows (query 4 kq + r) rescaled by their queries' corrections
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float cr = __shfl(corr, 4 * kq + r, 64);
#pragma unroll
        for (int db = 0; db < 8; ++db) O[db][r] *= cr;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {  // keys of sub-blocks 2j and 2j+1
        bf16x8_t phi, plo;
        split_bf16((f32x8_t){s[2 * j][0], s[2 * j][1], s[2 * j][2], s[2 * j][3],
                             s[2 * j + 1][0], s[2 * j + 1][1], s[2 * j + 1][2], s[2 * j + 1][3]}, phi, plo);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const uint2 w0 = *(const uint2 *)&vt[part][16 * db + ql][32 * j + 4 * kq];
          const uint2 w1 = *(const uint2 *)&vt[part][16 * db + ql][32 * j + 16 + 4 * kq];
          const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, make_uint4(w0.x, w0.y, w1.x, w1.y));
          O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, vb, O[db], 0, 0, 0);
          O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vb, O[db], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the next block's staging overwrites vt
  }
  // the parts merged in order (part 0's sums first), normalised, stored;
  // part 0 always holds block 0, whose keys every query sees
  if (part > 0) {
    if (kq == 0) {
      ml[part - 1][g][0][ql] = m_run;
      ml[part - 1][g][1][ql] = l_run;
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) mo[part - 1][g][db][lane] = O[db];
  }
  __syncthreads();
  if (part == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qq = 4 * kq + r;
      const float m0 = __shfl(m_run, qq, 64), l0 = __shfl(l_run, qq, 64);
      float m = m0;
#pragma unroll
      for (int q = 0; q < NPART - 1; ++q) m = fmaxf(m, ml[q][g][0][qq]);
      const float c0 = expf(m0 - m);
      float cp[NPART - 1];
      float L = l0 * c0;
#pragma unroll
      for (int q = 0; q < NPART - 1; ++q) {
        const float mq = ml[q][g][0][qq];
        cp[q] = mq == -INFINITY ? 0.f : expf(mq - m);
        L += ml[q][g][1][qq] * cp[q];
      }
      if (qq < nval) {
        float *op = a.o + (size_t)(row0 + qq) * a.nq * HD + (size_t)h * HD + ql;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          float o = O[db][r] * c0;
#pragma unroll
          for (int q = 0; q < NPART - 1; ++q) o += mo[q][g][db][lane][r] * cp[q];
          op[16 * db] = o / L;
        }
      }
    }
  }
}

hipError_t launch_attn_prompt(int hd, int kv_bf16, const AttnArgs &a, int n_streams, hipStream_t s) {
  const int G = a.nq / a.nkv;
  if (hd != 128 || !kv_bf16 || !a.rows.pf || a.qkv || !(G == 1 || G == 2)) return hipErrorInvalidValue;
  const dim3 grid(n_streams * ((a.rows.rows_per_slot + 15) / 16), a.nkv);
  if (G == 1) hipLaunchKernelGGL((attn_prompt_kernel<1>), grid, dim3(64 * PNPART), 0, s, a);
  else hipLaunchKernelGGL((attn_prompt_kernel<2>), grid, dim3(128 * PNPART), 0, s, a);
  return hipGetLastError();
}


// ------------------------------------------------------------------ batched projections (MFMA)
//
// y[M][N] = epi(x~ . W^T) for M <= GEMM_MAX_ROWS rows in 64-row blocks: x~ = bf16(x * rinv * gain) (or
// bf16(x)); weight rows in their storage format (bf16, or q8 / q4 codes
// converted exactly to bf16 with the 32-wide block scale applied to each
// block's product).
// v_mfma_f32_16x16x32_bf16 lane layout (checked on the device): A[16][32]
// row l%16, k (l/16)*8..+8; B[32][16] k (l/16)*8..+8, column l%16; D[16][16]
// c[j] at row (l/16)*4+j, column l%16.  A = 16 weight rows, B = 16 activation
// rows (transposed), so D[j] is the partial of y[m = l%16][n = (l/16)*4 + j].

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GT = 32;        // output columns per tile
constexpr int GBK = 256;      // K slice per workgroup
constexpr int GXS = GBK + 8;  // LDS row stride (bf16) of the staged operand: conflict-free B reads

// Weight row n of matrix `mat` (0: the segmented q|k|v or single matrix, 1:
// up).  The segment is chosen with selects on the kernel arguments: indexing
// a.seg[] with a computed index would read the argument block from memory
// before the first weight load could issue.
template <int WT>
__device__ __forceinline__ const uint8_t *gemm_row(const GemmArgs &a, int mat, int n, const uint16_t *&sc) {
  const void *w = a.up.w;
  const uint16_t *scb = a.up.sc;
  int r = n;
  if (mat == 0) {
    const bool s1 = a.nseg > 1 && n >= a.seg_end[0];
    const bool s2 = a.nseg > 2 && n >= a.seg_end[1];
    w = s2 ? a.seg[2].w : s1 ? a.seg[1].w : a.seg[0].w;
    scb = s2 ? a.seg[2].sc : s1 ? a.seg[1].sc : a.seg[0].sc;
    r = n - (s2 ? a.seg_end[1] : s1 ? a.seg_end[0] : 0);
  }
  sc = scb ? scb + (size_t)r * (a.K / 32) : nullptr;
  return (const uint8_t *)w + (size_t)r * row_bytes<WT>(a.K);
}

__device__ __forceinline__ uint32_t i8pair_bf16(uint32_t w, int b) {
  const float lo = (float)(int8_t)(w >> (8 * b)), hi = (float)(int8_t)(w >> (8 * b + 8));
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// 4-bit codes b and b + 1 of w as a bf16 pair (c - 8 is exact in bf16)
__device__ __forceinline__ uint32_t q4pair_bf16(uint32_t w, int b) {
  const float lo = (float)((int)((w >> (4 * b)) & 15u) - 8), hi = (float)((int)((w >> (4 * b + 4)) & 15u) - 8);
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// a lane's 8 consecutive weights of one 32-wide step: 16 bytes of bf16, 8 of
// int8 or 4 of 4-bit codes, and the same 8 as the MFMA's bf16 operand (block
// formats unscaled: the scale is applied to the product)
template <int WT> struct GemmW;
template <> struct GemmW<W_BF16> { typedef uint4 V; };
template <> struct GemmW<W_Q8> { typedef uint2 V; };
template <> struct GemmW<W_Q4> { typedef uint32_t V; };

template <int WT>
__device__ __forceinline__ bf16x8_t gemm_w_bf16(const typename GemmW<WT>::V w) {
  if constexpr (WT == W_BF16) {
    return __builtin_bit_cast(bf16x8_t, w);
  } else if constexpr (WT == W_Q8) {
    return __builtin_bit_cast(bf16x8_t, make_uint4(i8pair_bf16(w.x, 0), i8pair_bf16(w.x, 2),
                                                   i8pair_bf16(w.y, 0), i8pair_bf16(w.y, 2)));
  } else {
    return __builtin_bit_cast(bf16x8_t, make_uint4(q4pair_bf16(w, 0), q4pair_bf16(w, 2),
                                                   q4pair_bf16(w, 4), q4pair_bf16(w, 6)));
  }
}

// split-K partials are written and read back with 16-byte buffer accesses at
// agent scope (cache policy sc1), so the tile's last workgroup, on any XCD,
// reads what the others wrote
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(float *p) {
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, 0x7fffffff, 0x00020000);
}
constexpr int CPOL_SC1 = 16;

// Grid z: 64-row blocks of the activation rows, each its own workgroups (the
// blocks of one tile read the same weights; their ids differ by a multiple of
// 8, so they run on one XCD and share its L2).  KPW: consecutive 256-wide K
// slices per workgroup (grid y = K / 256 / KPW), accumulated in the MFMA
// registers slice after slice, so a tile has KPW times fewer split-K partials
// for its last workgroup to read back; every slice's loads are issued first.
template <int WT, int EPI, int KPW>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  // The tile's weight rows form NSUB blocks of 16; each block's K slice is
  // split over WPB waves, so every wave owns SPW 32-wide steps of one block
  // and loads them exactly once, then applies them to every 16-row activation
  // block.
  constexpr int NSUB = EPI == EPI_GATED ? 4 : 2;
  constexpr int WPB = 4 / NSUB;
  constexpr int SPW = GBK / 32 / WPB;
  constexpr int NBLK = GBK / 32;  // q8 / q4 scale blocks per weight row in the slice
  __shared__ __attribute__((aligned(16))) uint16_t xs[64 * GXS];
  __shared__ float rinv[64];
  __shared__ float gs[GBK];
  __shared__ float scl[w_blocked(WT) ? NSUB * 16 * NBLK : 1];
  __shared__ __attribute__((aligned(16))) f32x4_t red[WPB > 1 ? 4 * 64 * (NSUB * (WPB - 1)) : 1];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tn = blockIdx.x, ks = blockIdx.y, KS = gridDim.y;
  const int M = a.M, K = a.K, N = a.N;
  const int mb = 64 * blockIdx.z;                // first row of this block
  const int M0 = M - mb < 64 ? M - mb : 64;      // its rows
  const int MT = (M0 + 15) / 16;
  const int kw = ks * KPW * GBK;                 // first K column of this workgroup's slices
  const int NP = EPI == EPI_GATED ? 2 * N : N;  // partial columns (gated: gate then up)
  const __amdgpu_buffer_rsrc_t prs = part_rsrc(a.part);
  const int nb = wave / WPB, kq = wave % WPB;
  const int mat = EPI == EPI_GATED ? nb / 2 : 0;
  const int nrow0 = tn * GT + (EPI == EPI_GATED ? (nb % 2) : nb) * 16;

  // Loads first, in the order they are consumed, so that waiting for the
  // operand does not wait for the weights: the rows' sums of squares (thread
  // t sums row t / 4's slots t % 4, t % 4 + 4, ...), the gains, the operand
  // slices (eight columns per item), block scales, then the weights.  Every
  // load is unconditional, from a clamped in-bounds address, and masked where
  // it is used: a load under a branch makes the compiler wait for it at the
  // join.
  const int sm = tid >> 2, sq4 = tid & 3;
  const bool norm_row = a.gain && sm < M0;
  const float *ssp = a.gain ? a.ssq + (size_t)(mb + min(sm, M0 - 1)) * a.ssq_stride : a.x;
  float sqv[8];  // slots sq4 + 4 i, i < 8 (hidden widths up to 1024; wider rows add a loop)
#pragma unroll
  for (int i = 0; i < 8; ++i) sqv[i] = ssp[min(sq4 + 4 * i, K / 32 - 1)];
  // each slice's gain element as two 16-bit loads (bf16: the same half
  // twice); without a norm, row 0 of x stands in as an in-bounds address
  const uint16_t *gp = (const uint16_t *)(a.gain ? a.gain : (const void *)a.x);
  uint16_t glo[KPW], ghi[KPW];
#pragma unroll
  for (int j = 0; j < KPW; ++j) {
    const size_t gi = a.gain_bf16 ? (size_t)(kw + j * GBK + tid) : 2 * (size_t)(kw + j * GBK + tid);  // GBK == blockDim
    glo[j] = gp[gi];
    ghi[j] = gp[a.gain_bf16 ? gi : gi + 1];
  }
  constexpr int IT = 64 * (GBK / 8) / 256;
  float4 xv[KPW][IT][2];
#pragma unroll
  for (int j = 0; j < KPW; ++j)
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int e = tid + it * 256, m = e / (GBK / 8), c = e % (GBK / 8);
      if (it * 256 >= MT * 16 * (GBK / 8)) break;  // rows past the last 16-row block
      const float *xr = a.x + (size_t)(mb + min(m, M0 - 1)) * a.x_stride + kw + j * GBK + 8 * c;
      xv[j][it][0] = *(const float4 *)xr;
      xv[j][it][1] = *(const float4 *)(xr + 4);
    }
  constexpr int NSC = NSUB * 16 * NBLK / 256;  // block scales per thread and slice
  static_assert(NSUB * 16 * NBLK % 256 == 0 && 64 % NBLK == 0, "a wave's scales lie in one weight block");
  uint16_t sv[KPW][NSC];
  if constexpr (w_blocked(WT)) {
    // entry e: tile row r = e / NBLK (block r / 16, row r % 16 of it), scale
    // block e % NBLK; a wave's 64 entries are rows of one block
#pragma unroll
    for (int q = 0; q < NSC; ++q) {
      const int e = tid + 256 * q, r = e / NBLK, b = e % NBLK;
      const int rb = __builtin_amdgcn_readfirstlane(r / 16);
      const int rn0 = tn * GT + (EPI == EPI_GATED ? (rb % 2) : rb) * 16;
      const uint16_t *sp;
      (void)gemm_row<WT>(a, EPI == EPI_GATED ? rb / 2 : 0, rn0, sp);
#pragma unroll
      for (int j = 0; j < KPW; ++j) sv[j][q] = sp[(size_t)(r % 16) * (K / 32) + (kw + j * GBK) / 32 + b];
    }
  }
  typedef typename GemmW<WT>::V WVec;
  WVec wv[KPW][SPW];
  {
    // the block's 16 rows lie in one segment (segment ends are multiples of 16)
    const int n0 = __builtin_amdgcn_readfirstlane(nrow0);
    const uint16_t *sc;
    const uint8_t *wr = gemm_row<WT>(a, __builtin_amdgcn_readfirstlane(mat), n0, sc);
    const int n = n0 + (lane & 15);  // the weight row this lane loads
    wr += (size_t)(n < N ? lane & 15 : 0) * row_bytes<WT>(K);
#pragma unroll
    for (int j = 0; j < KPW; ++j)
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
        const int k = kw + j * GBK + (kq * SPW + s) * 32 + (lane >> 4) * 8;
        wv[j][s] = *(const WVec *)(wr + row_bytes<WT>(k));
      }
  }

  // RMSNorm row scales to LDS
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) sq += norm_row && sq4 + 4 * i < K / 32 ? sqv[i] : 0.f;
  if (norm_row)
    for (int i = sq4 + 32; i < K / 32; i += 4) sq += ssp[i];
  sq += __shfl_xor(sq, 1, 64);
  sq += __shfl_xor(sq, 2, 64);
  if (sq4 == 0) rinv[sm] = a.gain ? 1.0f / sqrtf(sq / (float)K + a.eps) : 1.f;

  // products of this wave's steps with every activation block, slice by slice
  f32x4_t acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KPW; ++j) {
    const int k0 = kw + j * GBK;
    if (j > 0) __syncthreads();  // every wave is done with the last slice's operand, gain and scales
    // the slice's gain and block scales to LDS
    gs[tid] = !a.gain ? 1.f : __uint_as_float(a.gain_bf16 ? (uint32_t)glo[j] << 16 : ((uint32_t)ghi[j] << 16) | glo[j]);
    if constexpr (w_blocked(WT))
#pragma unroll
      for (int q = 0; q < NSC; ++q) scl[tid + 256 * q] = f16_to_f32(sv[j][q]);
    __syncthreads();
    // operand slice in LDS as bf16: rows < MT * 16 (zero past M)
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int e = tid + it * 256, m = e / (GBK / 8), c = e % (GBK / 8);
      if (m >= MT * 16) break;
      float v[8] = {xv[j][it][0].x, xv[j][it][0].y, xv[j][it][0].z, xv[j][it][0].w,
                    xv[j][it][1].x, xv[j][it][1].y, xv[j][it][1].z, xv[j][it][1].w};
      uint4 o = make_uint4(0u, 0u, 0u, 0u);
      if (m < M0) {
        if (a.gain) {
          const float r = rinv[m];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = v[i] * r * gs[8 * c + i];
          if (a.normed_out && tn == 0)
#pragma unroll
            for (int i = 0; i < 8; ++i) a.normed_out[(size_t)(mb + m) * K + k0 + 8 * c + i] = v[i];
        }
        o.x = (uint32_t)bf16_bits(v[0]) | ((uint32_t)bf16_bits(v[1]) << 16);
        o.y = (uint32_t)bf16_bits(v[2]) | ((uint32_t)bf16_bits(v[3]) << 16);
        o.z = (uint32_t)bf16_bits(v[4]) | ((uint32_t)bf16_bits(v[5]) << 16);
        o.w = (uint32_t)bf16_bits(v[6]) | ((uint32_t)bf16_bits(v[7]) << 16);
      }
      *(uint4 *)&xs[m * GXS + 8 * c] = o;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int kl = (kq * SPW + s) * 32;  // step's offset in the slice
      const bf16x8_t av = gemm_w_bf16<WT>(wv[j][s]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt >= MT) break;
        const uint4 bx = *(const uint4 *)&xs[(mt * 16 + (lane & 15)) * GXS + kl + (lane >> 4) * 8];
        const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, bx);
        if constexpr (WT == W_BF16) {
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[mt], 0, 0, 0);
        } else {
          const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
          const f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, zero, 0, 0, 0);
          const float *sr = &scl[(nb * 16 + (lane >> 4) * 4) * NBLK + kl / 32];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[mt][q] += t[q] * sr[q * NBLK];
        }
      }
    }
  }
  // waves of one block sum their K parts (lower K part first)
  if constexpr (WPB > 1) {
    if (kq > 0)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        if (mt < MT) red[((nb * (WPB - 1) + kq - 1) * 4 + mt) * 64 + lane] = acc[mt];
    __syncthreads();
    if (kq == 0)
#pragma unroll
      for (int q = 1; q < WPB; ++q)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          if (mt < MT) acc[mt] += red[((nb * (WPB - 1) + q - 1) * 4 + mt) * 64 + lane];
  }
  // this lane's four partials are four consecutive columns of row m
  if (kq == 0) {
    const int nj = nrow0 + (lane >> 4) * 4;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int m = mt * 16 + (lane & 15);
      if (mt < MT && m < M0 && nj < N)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u_t, acc[mt]), prs,
                                               (int)((((size_t)ks * M + mb + m) * NP + (mat ? N : 0) + nj) * 4), 0,
                                               CPOL_SC1);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are acknowledged
  __syncthreads();
  if (tid == 0) {
    uint32_t *cn = a.cnt + blockIdx.z * gridDim.x + tn;
    const uint32_t old = __hip_atomic_fetch_add(cn, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == (uint32_t)(KS - 1);
    if (last) __hip_atomic_store(cn, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;

  // the tile's last workgroup: sum the K slices in order, then the epilogue;
  // thread t covers row t / 4, columns (t % 4) * 8 .. + 8 of the tile.  The
  // residual row and every slice of a group (all of them for K <= 3072) are
  // requested before the first sum, so the epilogue waits for one round trip.
  {  // this block's rows
    const int m = mb + (tid >> 2), c0 = (tid & 3) * 8;
    const int nb0 = tn * GT + c0;
    sq = 0.f;
    if (m < M && nb0 < N) {
      float *yr = a.y + (size_t)m * a.y_stride + nb0;
      float yv[8];
      if constexpr (EPI == EPI_RESID)
#pragma unroll
        for (int i = 0; i < 8; ++i) yv[i] = yr[i];
      float g8[8], u8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) g8[i] = u8[i] = 0.f;
      constexpr int QG = EPI == EPI_GATED ? 6 : 12;  // slices per group
      for (int q0 = 0; q0 < KS; q0 += QG) {
        f32x4v_t lg[QG][2], lu[EPI == EPI_GATED ? QG : 1][2];
#pragma unroll
        for (int qq = 0; qq < QG; ++qq)
          if (q0 + qq < KS) {
            const int off = (int)((((size_t)(q0 + qq) * M + m) * NP + nb0) * 4);
            lg[qq][0] = __builtin_bit_cast(f32x4v_t, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, CPOL_SC1));
            lg[qq][1] = __builtin_bit_cast(f32x4v_t, __builtin_amdgcn_raw_buffer_load_b128(prs, off + 16, 0, CPOL_SC1));
            if constexpr (EPI == EPI_GATED) {
              lu[qq][0] = __builtin_bit_cast(f32x4v_t, __builtin_amdgcn_raw_buffer_load_b128(prs, off + N * 4, 0, CPOL_SC1));
              lu[qq][1] = __builtin_bit_cast(f32x4v_t, __builtin_amdgcn_raw_buffer_load_b128(prs, off + N * 4 + 16, 0, CPOL_SC1));
            }
          }
#pragma unroll
        for (int qq = 0; qq < QG; ++qq)
          if (q0 + qq < KS)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              g8[i] += lg[qq][i >> 2][i & 3];
              if constexpr (EPI == EPI_GATED) u8[i] += lu[qq][i >> 2][i & 3];
            }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int n = nb0 + i;
        const float g = g8[i], u = u8[i];
        if constexpr (EPI == EPI_STORE) {
          yr[i] = g;
        } else if constexpr (EPI == EPI_RESID) {
          const float v = yv[i] + g;
          yr[i] = v;
          if (a.copy_out) a.copy_out[(size_t)m * a.copy_stride + n] = v;
          sq += v * v;
        } else {
          yr[i] = silu(g) * u;
        }
      }
    }
    if (EPI == EPI_RESID && a.ssq_out) {
      sq += __shfl_xor(sq, 1, 64);
      sq += __shfl_xor(sq, 2, 64);
      if ((tid & 3) == 0 && m < M) a.ssq_out[(size_t)m * (N / 32) + tn] = sq;
    }
  }
}

template <int WT, int KPW>
static hipError_t gemm_kpw(int epi, const GemmArgs &a, hipStream_t s) {
  const dim3 grid((a.N + GT - 1) / GT, a.K / GBK / KPW, (a.M + 63) / 64);
  if (epi == EPI_STORE) hipLaunchKernelGGL((gemm_kernel<WT, EPI_STORE, KPW>), grid, dim3(256), 0, s, a);
  else if (epi == EPI_RESID) hipLaunchKernelGGL((gemm_kernel<WT, EPI_RESID, KPW>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((gemm_kernel<WT, EPI_GATED, KPW>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
template <int WT>
static hipError_t gemm_wt(int epi, const GemmArgs &a, hipStream_t s) {
  return a.kpw == 2 ? gemm_kpw<WT, 2>(epi, a, s) : gemm_kpw<WT, 1>(epi, a, s);
}

hipError_t launch_gemm(int wtype, int epi, const GemmArgs &a, hipStream_t s) {
  if (a.M < 1 || a.M > GEMM_MAX_ROWS || a.K % GBK || a.N % GT || a.nseg < 1 || a.nseg > 3) return hipErrorInvalidValue;
  if (a.kpw < 0 || a.kpw > 2 || (a.K / GBK) % (a.kpw > 1 ? a.kpw : 1)) return hipErrorInvalidValue;
  for (int i = 0; i + 1 < a.nseg; ++i)  // a 16-row weight block never straddles two segments
    if (a.seg_end[i] % 16) return hipErrorInvalidValue;
  if (wtype == W_BF16) return gemm_wt<W_BF16>(epi, a, s);
  if (wtype == W_Q8) return gemm_wt<W_Q8>(epi, a, s);
  if (wtype == W_Q4) return gemm_wt<W_Q4>(epi, a, s);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ row sums of squares
//
// Producers of residual rows also leave the rows' sums of squares in 32-column
// slots ([row][H/32]) for the batched projections' RMSNorm.  A block covering
// columns [c0, c0 + n) writes its sum into slot c0/32 and zeros into the other
// slots it covers.
__device__ __forceinline__ void put_ssq(float *ssq, int H, int row, int c0, int n, float v) {
  __shared__ float red[4];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const int ns = (n + 31) / 32;
  if ((int)threadIdx.x < ns)
    ssq[(size_t)row * (H / 32) + c0 / 32 + threadIdx.x] =
        threadIdx.x == 0 ? (red[0] + red[1]) + (red[2] + red[3]) : 0.f;
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
  if (a.ssq) {
    float v = 0.f;
    if (i < a.H) v = a.x[(size_t)r * a.H + i];
    put_ssq(a.ssq, a.H, r, blockIdx.y * 256, min(256, a.H - (int)blockIdx.y * 256), v * v);
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
  float v0 = 0.f, v1 = 0.f;
  if (i < a.H) {
    v0 = a.bridge[(size_t)b * a.H + i];
    v1 = tab_at(a.code_emb, a.tab_bf16, (size_t)c * a.H + i);
    a.x[(size_t)(2 * b) * a.H + i] = v0;
    a.x[(size_t)(2 * b + 1) * a.H + i] = v1;
  }
  if (a.ssq) {
    const int n = min(256, a.H - (int)blockIdx.y * 256);
    put_ssq(a.ssq, a.H, 2 * b, blockIdx.y * 256, n, v0 * v0);
    __syncthreads();
    put_ssq(a.ssq, a.H, 2 * b + 1, blockIdx.y * 256, n, v1 * v1);
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

// Logit -> unsigned key in the same order (-0 and +0 equal, as they compare).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x == 0.f ? 0.f : x);
  return b ^ ((b >> 31) ? 0xffffffffu : 0x80000000u);
}

// This thread's best sampled score among the top_k largest of Vc <= 2048
// logits (logit i = u * 256 + tid is value u of the thread): the k-th largest
// key by a radix select, 8 bits per pass from the top, over LDS histograms;
// logits equal to it count in index order, lower indices first (the argmax's
// tie rule).  Every other logit scores -inf.  256 threads, all of them.
__device__ __forceinline__ void top_k_scan(const float *lg, int Vc, int k, float inv_temp, uint64_t seed, int slot,
                                           int q, int jc, float &best, int &bi) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel[2];      // key prefix found so far, members still to place
  __shared__ uint32_t eqc[8][4];   // logits equal to the threshold per (value slot, wave)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float v[8];
  uint32_t key[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    v[u] = lg[min(u * 256 + tid, Vc - 1)];
    key[u] = order_key(v[u]);
  }
  uint32_t prefix = 0, need = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hmask = pass ? 0xffffffffu << (shift + 8) : 0u;
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u * 256 + tid < Vc && (key[u] & hmask) == prefix) atomicAdd(&hist[(key[u] >> shift) & 255], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 255 - 4l .. 252 - 4l (descending); inclusive scan over lanes
      uint32_t c[4], c4 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) { c[e] = hist[255 - 4 * lane - e]; c4 += c[e]; }
      uint32_t cum = c4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(cum, o, 64);
        if (lane >= o) cum += t;
      }
      const uint64_t hit = __ballot(cum >= need);
      if (lane == (int)__ffsll((unsigned long long)hit) - 1) {  // the lane whose bins reach the k-th
        uint32_t run = cum - c4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (run + c[e] >= need) {
            sel[0] = prefix | ((uint32_t)(255 - 4 * lane - e) << shift);
            sel[1] = need - run;
            break;
          }
          run += c[e];
        }
      }
    }
    __syncthreads();
    prefix = sel[0];
    need = sel[1];
  }
  // logits equal to the threshold key: the first `need` in index order are members
  if (lane == 0)
#pragma unroll
    for (int u = 0; u < 8; ++u) eqc[u][wave] = 0;
  uint64_t eqm[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    eqm[u] = __ballot(u * 256 + tid < Vc && key[u] == prefix);
    if (lane == 0) eqc[u][wave] = (uint32_t)__popcll(eqm[u]);
  }
  __syncthreads();
  uint32_t before = 0;  // equal logits at lower indices than value slot u of this thread
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = u * 256 + tid;
    uint32_t rank = before;
    for (int w = 0; w < wave; ++w) rank += eqc[u][w];
    rank += (uint32_t)__popcll(eqm[u] & ((1ull << lane) - 1ull));
    for (int w = 0; w < 4; ++w) before += eqc[u][w];
    const bool member = i < Vc && (key[u] > prefix || (key[u] == prefix && rank < need));
    const float s = member ? sample_score(v[u], inv_temp, seed, slot, q, jc, i) : -INFINITY;
    if (member && s > best) { best = s; bi = i; }
  }
}

__global__ __launch_bounds__(256) void argmax_kernel(ArgmaxArgs a) {
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *lg = a.logits + (size_t)r * a.Vc;
  // The code's sampling key: stream, frame position, index in the frame
  const float inv_temp = __int_as_float(a.ctl[2]);
  const uint64_t seed = (uint64_t)(uint32_t)a.ctl[3] | ((uint64_t)(uint32_t)a.ctl[4] << 32);
  const int top_k = a.ctl[5];
  int slot = r, q, jc = 0;
  if (a.mode == AM_PREFILL) {
    if (a.ctl[PF_HEAD + r] < 0) return;  // this stream's prompt goes on in the next chunk
    slot = a.ctl[PF_SLOT + r];
    q = a.ctl[PF_T + r];
    for (int i = tid; i < a.H; i += 256) a.bridge[(size_t)slot * a.H + i] = a.bridge_src[(size_t)r * a.H + i];
    for (int i = tid; i < a.Vc; i += 256) a.logits_out[(size_t)slot * a.Vc + i] = lg[i];
  } else {
    q = a.mode == AM_PRED ? a.pos[r] : a.pos[r] + 1;
    jc = a.mode == AM_PRED ? a.j + 1 : 0;
  }
  const bool sampled = inv_temp != 0.f;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  if (sampled && top_k > 0 && top_k < a.Vc) {
    top_k_scan(lg, a.Vc, top_k, inv_temp, seed, slot, q, jc, best, bi);
  } else {
    // Eight logits per thread in flight at a time (a plain loop waits on each
    // load); the first group is outside any loop.
    auto scan = [&](int i0) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = lg[min(i0 + u * 256 + tid, a.Vc - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 256 + tid;
        const float s = sampled ? sample_score(v[u], inv_temp, seed, slot, q, jc, i) : v[u];
        if (i < a.Vc && s > best) { best = s; bi = i; }  // increasing i: first max kept
      }
    };
    scan(0);
    for (int i0 = 8 * 256; i0 < a.Vc; i0 += 8 * 256) scan(i0);
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
      a.c0_state[slot] = b;
      a.pos[slot] = q;
    }
    code = c;
  }
  if (a.mode == AM_PRED && a.x_next && a.j + 2 < a.G) {
    __syncthreads();
    const int c = code;
    const size_t base = ((size_t)(a.j + 1) * a.Vc + c) * a.H;
    float sq = 0.f;
    for (int i0 = 0; i0 < a.H; i0 += 4 * 256) {  // four loads in flight per thread
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = tab_at(a.code_emb, a.tab_bf16, base + min(i0 + u * 256 + tid, a.H - 1));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * 256 + tid;
        if (i < a.H) {
          a.x_next[(size_t)r * a.H + i] = v[u];
          sq += v[u] * v[u];
        }
      }
    }
    if (a.ssq) put_ssq(a.ssq, a.H, r, 0, a.H, sq);
  }
}

__global__ __launch_bounds__(256) void pf_rows_kernel(const int32_t *pf, const float *x, float *xh, int32_t H) {
  const int i = blockIdx.x, src = max(pf[PF_HEAD + i], 0);
  for (int k = threadIdx.x; k < H; k += 256) xh[(size_t)i * H + k] = x[(size_t)src * H + k];
}

hipError_t launch_pf_rows(const int32_t *pf, const float *x, float *xh, int32_t n, int32_t H, hipStream_t s) {
  hipLaunchKernelGGL(pf_rows_kernel, dim3(n), dim3(256), 0, s, pf, x, xh, H);
  return hipGetLastError();
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

// Plain streaming read of n16 16-byte chunks: a grid-stride loop with four
// 16-byte loads in flight per thread, the words folded by xor so the loads
// stay live; each thread stores its fold to sink (the achievable-bandwidth
// reference the frame kernels are measured against).
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ src, size_t n16,
                                                          uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

hipError_t launch_stream_read(const void *src, size_t bytes, void *sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamGrid), dim3(256), 0, s, (const uint4 *)src, bytes / 16,
                     (uint32_t *)sink);
  return hipGetLastError();
}

}  // namespace qtk
