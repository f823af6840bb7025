// exchange_probe.hip -- latency of the tagged-word exchanges the persistent
// frame kernel is built on, measured with one workgroup per compute unit
// (a cooperative launch, so all are resident; placement is read back from
// the XCC_ID hardware register).  Every wait is bounded: a timed-out wait
// raises an error flag and every workgroup leaves.  Build and run with
// `python -m autoregressive_codebook_tts_frame_amd.exchange_probe`.
//
// Modes (N = words exchanged per round):
//   0  all-to-all: each workgroup publishes N / nwg contiguous words (8-byte
//      tag | value at agent scope) and polls all N
//   3  ping-pong of one word between workgroup 0 and a peer, agent scope
//   4  ping-pong on one XCD through its L2: non-temporal stores and loads
//   1  XCD relay: each XCD's workgroups poll one slice each at agent scope and
//      re-publish it into an XCD-local copy (L2), which every workgroup polls
//   5  all-to-all with two load sets per word in flight
//   9  all-to-all, each workgroup's share on its own 64-byte sector
//  12  all-to-all among the 32 workgroups of one XCD, through its L2
//  13  every workgroup polls 8 vectors of N words, one published by each XCD
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#define NT 320
#define PER 8
#define SPIN_LIMIT (1u << 20)

struct A {
  uint64_t *g;    // [2][N]
  uint64_t *loc;  // [8][2][N]
  int N, rounds, mode, nwg, peer;
  int *err;
  unsigned *xcnt;  // [8]
  unsigned *bar;
  long long *t;  // [4]
  int *xcc;      // [nwg]
  int *bad;
  uint32_t base;
};

__device__ __forceinline__ uint64_t ld_agent(const uint64_t *p) {
  return __hip_atomic_load((uint64_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_wg(const uint64_t *p) {
  uint64_t v;  // nt: misses L1, hits the XCD's L2; waits in the same block
  asm volatile("global_load_dwordx2 %0, %1, off nt\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}
// eight nt loads in flight, waited for in the same block
__device__ __forceinline__ void ld8_wg(const uint64_t *const *p, uint64_t *v) {
  asm volatile(
      "global_load_dwordx2 %0, %8, off nt\n\t"
      "global_load_dwordx2 %1, %9, off nt\n\t"
      "global_load_dwordx2 %2, %10, off nt\n\t"
      "global_load_dwordx2 %3, %11, off nt\n\t"
      "global_load_dwordx2 %4, %12, off nt\n\t"
      "global_load_dwordx2 %5, %13, off nt\n\t"
      "global_load_dwordx2 %6, %14, off nt\n\t"
      "global_load_dwordx2 %7, %15, off nt\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
      : "memory");
}
__device__ __forceinline__ void st_agent(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_wg(uint64_t *p, uint64_t v) {
  __builtin_nontemporal_store(v, p);
}
__device__ __forceinline__ int err_get(int *e) {
  return __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void err_set(int *e) { __hip_atomic_store(e, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ uint32_t val(uint32_t r, uint32_t i) { return i * 2654435761u + r * 40503u; }

// poll words [lo, hi) of src until each has tag; checks values; then
// optionally forwards each word to dst (workgroup-scope store).  All threads.
template <bool AGENT, bool FWD>
__device__ bool poll(const A &a, const uint64_t *src, int lo, int hi, uint32_t tag, uint32_t r, uint64_t *dst,
                     int &nbad) {
  for (int b0 = lo; b0 < hi; b0 += PER * NT) {
    uint64_t v[PER];
    const uint64_t *ad[PER];
    uint32_t pend = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = b0 + (int)threadIdx.x + k * NT;
      ad[k] = src + (i < hi ? i : hi - 1);  // in bounds; the tail is ignored
      if (i < hi) pend |= 1u << k;
    }
    if (!pend) continue;
    for (uint32_t spins = 0;; ++spins) {
      if (AGENT) {
#pragma unroll
        for (int k = 0; k < PER; ++k)
          if ((pend >> k) & 1u) v[k] = ld_agent(ad[k]);
      } else {
        ld8_wg(ad, v);
      }
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if (((pend >> k) & 1u) && (uint32_t)(v[k] >> 32) == tag) {
          const int i = b0 + (int)threadIdx.x + k * NT;
          if ((uint32_t)v[k] != val(r, i)) ++nbad;
          if (FWD) st_wg(dst + i, v[k]);
          pend &= ~(1u << k);
        }
      if (!pend) break;
      if (spins > SPIN_LIMIT || ((spins & 255u) == 255u && err_get(a.err))) {
        err_set(a.err);
        return false;
      }
    }
  }
  return true;
}

// Two load sets per word in flight (issued SLP sleep units apart): a word's
// arrival is seen about half a round trip sooner.  Words tid + k NT, k < 4.
template <int SLP>
__device__ bool poll2(const A &a, const uint64_t *src, int n, uint32_t tag, uint32_t r, int &nbad) {
  const uint64_t *ad[4];
  uint32_t pend = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = (int)threadIdx.x + k * NT;
    ad[k] = src + (i < n ? i : n - 1);
    if (i < n) pend |= 1u << k;
  }
  if (!pend) return true;
  uint64_t va[4], vb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) va[k] = ld_agent(ad[k]);
  if (SLP) __builtin_amdgcn_s_sleep(SLP);
#pragma unroll
  for (int k = 0; k < 4; ++k) vb[k] = ld_agent(ad[k]);
  for (uint32_t spins = 0;; ++spins) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (((pend >> k) & 1u) && (uint32_t)(va[k] >> 32) == tag) {
        if ((uint32_t)va[k] != val(r, (int)threadIdx.x + k * NT)) ++nbad;
        pend &= ~(1u << k);
      }
    if (!pend) break;
#pragma unroll
    for (int k = 0; k < 4; ++k) va[k] = ld_agent(ad[k]);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (((pend >> k) & 1u) && (uint32_t)(vb[k] >> 32) == tag) {
        if ((uint32_t)vb[k] != val(r, (int)threadIdx.x + k * NT)) ++nbad;
        pend &= ~(1u << k);
      }
    if (!pend) break;
#pragma unroll
    for (int k = 0; k < 4; ++k) vb[k] = ld_agent(ad[k]);
    if (spins > SPIN_LIMIT || ((spins & 255u) == 255u && err_get(a.err))) {
      err_set(a.err);
      return false;
    }
  }
  return true;
}

// poll a padded vector: word j of workgroup w's share is at w * stride + j
__device__ bool poll_pad(const A &a, const uint64_t *src, int per, int stride, uint32_t tag, uint32_t r, int &nbad) {
  const int n = per * a.nwg;
  for (int b0 = 0; b0 < n; b0 += PER * NT) {
    uint64_t v[PER];
    const uint64_t *ad[PER];
    uint32_t pend = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = b0 + (int)threadIdx.x + k * NT;
      const int ii = i < n ? i : n - 1;
      ad[k] = src + (ii / per) * stride + ii % per;
      if (i < n) pend |= 1u << k;
    }
    if (!pend) continue;
    for (uint32_t spins = 0;; ++spins) {
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if ((pend >> k) & 1u) v[k] = ld_agent(ad[k]);
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if (((pend >> k) & 1u) && (uint32_t)(v[k] >> 32) == tag) {
          if ((uint32_t)v[k] != val(r, b0 + (int)threadIdx.x + k * NT)) ++nbad;
          pend &= ~(1u << k);
        }
      if (!pend) break;
      if (spins > SPIN_LIMIT || ((spins & 255u) == 255u && err_get(a.err))) {
        err_set(a.err);
        return false;
      }
    }
  }
  return true;
}

// poll n words of an XCD-local buffer with nt loads (asm, waited in-block)
__device__ bool poll_local(const A &a, const uint64_t *src, int n, uint32_t tag, int &nbad, uint32_t r) {
  for (int b0 = 0; b0 < n; b0 += PER * NT) {
    uint64_t v[PER];
    const uint64_t *ad[PER];
    uint32_t pend = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = b0 + (int)threadIdx.x + k * NT;
      ad[k] = src + (i < n ? i : n - 1);
      if (i < n) pend |= 1u << k;
    }
    if (!pend) continue;
    for (uint32_t spins = 0;; ++spins) {
      ld8_wg(ad, v);
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if (((pend >> k) & 1u) && (uint32_t)(v[k] >> 32) == tag) {
          if ((uint32_t)v[k] != val(r, b0 + (int)threadIdx.x + k * NT)) ++nbad;
          pend &= ~(1u << k);
        }
      if (!pend) break;
      if (spins > SPIN_LIMIT || ((spins & 255u) == 255u && err_get(a.err))) {
        err_set(a.err);
        return false;
      }
    }
  }
  return true;
}

__global__ __launch_bounds__(NT) void xbench(A a) {
  __shared__ int sh_abort, sh_li, sh_nx, sh_x;
  const int wg = blockIdx.x, tid = threadIdx.x;
  int nbad = 0;
  if (tid == 0) {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    x &= 7u;
    sh_x = (int)x;
    a.xcc[wg] = (int)x;
    sh_li = (int)atomicAdd(a.xcnt + x, 1u);
    sh_abort = 0;
    // grid barrier (every workgroup is resident: cooperative launch)
    __hip_atomic_fetch_add(a.bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (__hip_atomic_load(a.bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)a.nwg) {
      if (++spins > SPIN_LIMIT) { err_set(a.err); sh_abort = 1; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    sh_nx = (int)__hip_atomic_load(a.xcnt + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (sh_abort) return;
  const int x = sh_x, li = sh_li, nx = sh_nx;
  const int N = a.N;
  uint64_t *loc = a.loc + (size_t)x * 2 * N;

  if (a.mode == 3) {
    // ping-pong: g[0] written by wg 0, g[1] by the peer
    if (wg != 0 && wg != a.peer) return;
    if (tid != 0) return;
    const long long t0 = wall_clock64();
    for (int r = 0; r < a.rounds; ++r) {
      const uint32_t tag = a.base + r;
      if (wg == 0) {
        st_agent(a.g, ((uint64_t)tag << 32) | 7u);
        uint32_t spins = 0;
        while ((uint32_t)(ld_agent(a.g + 1) >> 32) != tag)
          if (++spins > SPIN_LIMIT) { err_set(a.err); return; }
      } else {
        uint32_t spins = 0;
        while ((uint32_t)(ld_agent(a.g) >> 32) != tag)
          if (++spins > SPIN_LIMIT) { err_set(a.err); return; }
        st_agent(a.g + 1, ((uint64_t)tag << 32) | 9u);
      }
    }
    if (wg == 0) { a.t[0] = t0; a.t[1] = wall_clock64(); }
    return;
  }
  if (a.mode == 4) {
    // ping-pong at workgroup scope (same XCD only)
    if (wg != 0 && wg != a.peer) return;
    if (tid != 0) return;
    const long long t0 = wall_clock64();
    for (int r = 0; r < a.rounds; ++r) {
      const uint32_t tag = a.base + r;
      if (wg == 0) {
        st_wg(a.g, ((uint64_t)tag << 32) | 7u);
        uint32_t spins = 0;
        while ((uint32_t)(ld_wg(a.g + 16) >> 32) != tag)
          if (++spins > SPIN_LIMIT) { err_set(a.err); return; }
      } else {
        uint32_t spins = 0;
        while ((uint32_t)(ld_wg(a.g) >> 32) != tag)
          if (++spins > SPIN_LIMIT) { err_set(a.err); return; }
        st_wg(a.g + 16, ((uint64_t)tag << 32) | 9u);
      }
    }
    if (wg == 0) { a.t[0] = t0; a.t[1] = wall_clock64(); }
    return;
  }

  long long t0 = 0;
  if (wg == 0 && tid == 0) t0 = wall_clock64();
  for (int r = 0; r < a.rounds; ++r) {
    const uint32_t tag = a.base + r;
    // two buffers, alternating: a word is rewritten two rounds later, after
    // every workgroup has consumed the round in between (so also this one)
    uint64_t *gb = a.g + (size_t)(r & 1) * N, *lb = loc + (size_t)(r & 1) * N;
    bool ok;
    if (a.mode == 12) {
      // XCD-local all-to-all: the nx workgroups of XCD x publish N words
      // into that XCD's buffer (nt stores: the XCD's L2) and poll all of it
      uint64_t *lb2 = loc + (size_t)(r & 1) * N;
      const int p0 = (int)((long long)li * N / nx), p1 = (int)((long long)(li + 1) * N / nx);
      for (int i = p0 + tid; i < p1; i += NT) st_wg(lb2 + i, ((uint64_t)tag << 32) | val(r, i));
      ok = poll_local(a, lb2, N, tag, nbad, r);
      if (!ok) sh_abort = 1;
      __syncthreads();
      if (sh_abort) break;
      continue;
    }
    if (a.mode == 13) {
      // cross-XCD partial vectors: XCD x's workgroups publish its vector of N
      // words (32-word shares), every workgroup polls all 8 vectors
      uint64_t *pb = a.g + (size_t)(r & 1) * 8 * 1024;
      uint64_t *mine = pb + (size_t)x * 1024;
      const int p0 = li * (N / nx), p1 = (li + 1) * (N / nx);
      for (int i = p0 + tid; i < p1; i += NT) st_agent(mine + i, ((uint64_t)tag << 32) | val(r, x * 1024 + i));
      // poll words x' * 1024 + i for i < N
      ok = true;
      {
        const int n = 8 * N;
        for (int b0 = 0; b0 < n && ok; b0 += PER * NT) {
          uint64_t v[PER];
          const uint64_t *ad[PER];
          uint32_t pend = 0;
#pragma unroll
          for (int k = 0; k < PER; ++k) {
            const int i = b0 + tid + k * NT;
            const int ii = i < n ? i : n - 1;
            ad[k] = pb + (size_t)(ii / N) * 1024 + ii % N;
            if (i < n) pend |= 1u << k;
          }
          if (!pend) continue;
          for (uint32_t spins = 0;; ++spins) {
#pragma unroll
            for (int k = 0; k < PER; ++k)
              if ((pend >> k) & 1u) v[k] = ld_agent(ad[k]);
#pragma unroll
            for (int k = 0; k < PER; ++k)
              if (((pend >> k) & 1u) && (uint32_t)(v[k] >> 32) == tag) pend &= ~(1u << k);
            if (!pend) break;
            if (spins > SPIN_LIMIT || ((spins & 255u) == 255u && err_get(a.err))) {
              err_set(a.err);
              ok = false;
              break;
            }
          }
        }
      }
      if (!ok) sh_abort = 1;
      __syncthreads();
      if (sh_abort) break;
      continue;
    }
    if (a.mode == 9) {
      // N / nwg words per workgroup, each share on sectors of its own
      const int per = N / a.nwg, stride = (per + 7) & ~7;
      uint64_t *pb = a.g + (size_t)(r & 1) * a.nwg * 16;
      for (int j = tid; j < per; j += NT) st_agent(pb + wg * stride + j, ((uint64_t)tag << 32) | val(r, wg * per + j));
      ok = poll_pad(a, pb, per, stride, tag, r, nbad);
      if (!ok) sh_abort = 1;
      __syncthreads();
      if (sh_abort) break;
      continue;
    }
    // publish this workgroup's share
    const int p0 = (int)((long long)wg * N / a.nwg), p1 = (int)((long long)(wg + 1) * N / a.nwg);
    for (int i = p0 + tid; i < p1; i += NT) st_agent(gb + i, ((uint64_t)tag << 32) | val(r, i));
    if (a.mode == 0) {
      ok = poll<true, false>(a, gb, 0, N, tag, r, nullptr, nbad);
    } else if (a.mode == 5) {
      ok = poll2<0>(a, gb, N, tag, r, nbad);
    } else {
      // slices of whole 128-byte lines: a line of the local copy has one writer
      const int nl = (N + 15) / 16;
      const int s0 = min(N, 16 * (int)((long long)li * nl / nx)), s1 = min(N, 16 * (int)((long long)(li + 1) * nl / nx));
      ok = poll<true, true>(a, gb, s0, s1, tag, r, lb, nbad);
      ok = ok && poll<false, false>(a, lb, 0, N, tag, r, nullptr, nbad);
    }
    if (!ok) sh_abort = 1;
    __syncthreads();
    if (sh_abort) break;
  }
  if (wg == 0 && tid == 0) { a.t[0] = t0; a.t[1] = wall_clock64(); }
  if (nbad) atomicAdd(a.bad, nbad);
}

#define CK(x)                                                                  \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

int main(int argc, char **argv) {
  int ncu = 0, coop = 0;
  CK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0));
  CK(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, 0));
  printf("CUs %d, cooperative launch %d\n", ncu, coop);
  if (!coop) return 1;
  const int maxN = 16384;
  uint64_t *g, *loc;
  int *err, *xcc, *bad;
  unsigned *xcnt, *bar;
  long long *t;
  CK(hipMalloc(&g, maxN * 8));
  CK(hipMalloc(&loc, 8 * maxN * 8));
  CK(hipMalloc(&err, 4));
  CK(hipMalloc(&xcc, 4 * 1024));
  CK(hipMalloc(&bad, 4));
  CK(hipMalloc(&xcnt, 4 * 8));
  CK(hipMalloc(&bar, 4));
  CK(hipMalloc(&t, 8 * 4));
  CK(hipMemset(g, 0, maxN * 8));
  CK(hipMemset(loc, 0, 8 * maxN * 8));
  int occ = 0;
  CK(hipFuncSetAttribute((const void *)xbench, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024));
  CK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, xbench, NT, 96 * 1024));
  printf("occupancy %d blocks/CU at %d threads\n", occ, NT);
  uint32_t base = 1;
  auto run = [&](int mode, int N, int rounds, int peer, bool print_xcc) {
    A a;
    a.g = g; a.loc = loc; a.N = N; a.rounds = rounds; a.mode = mode; a.nwg = ncu; a.peer = peer;
    a.err = err; a.xcnt = xcnt; a.bar = bar; a.t = t; a.xcc = xcc; a.bad = bad; a.base = base;
    base += rounds + 16;
    CK(hipMemset(err, 0, 4));
    CK(hipMemset(bad, 0, 4));
    CK(hipMemset(xcnt, 0, 32));
    CK(hipMemset(bar, 0, 4));
    CK(hipMemset(t, 0, 32));
    void *args[] = {&a};
    CK(hipLaunchCooperativeKernel((const void *)xbench, dim3(ncu), dim3(NT), args, 96 * 1024, 0));
    CK(hipDeviceSynchronize());
    int he = 0, hb = 0;
    long long ht[2];
    CK(hipMemcpy(&he, err, 4, hipMemcpyDeviceToHost));
    CK(hipMemcpy(&hb, bad, 4, hipMemcpyDeviceToHost));
    CK(hipMemcpy(ht, t, 16, hipMemcpyDeviceToHost));
    if (print_xcc) {
      std::vector<int> hx(ncu);
      CK(hipMemcpy(hx.data(), xcc, 4 * ncu, hipMemcpyDeviceToHost));
      int cnt[8] = {0};
      int rr = 1;
      for (int i = 0; i < ncu; ++i) { cnt[hx[i] & 7]++; if (hx[i] != i % 8) rr = 0; }
      printf("XCC counts:");
      for (int i = 0; i < 8; ++i) printf(" %d", cnt[i]);
      printf("; wg %% 8 == xcc for all: %d; first 16:", rr);
      for (int i = 0; i < 16; ++i) printf(" %d", hx[i]);
      printf("\n");
    }
    const double us = (ht[1] - ht[0]) / 100.0;  // 100 MHz
    printf("| %d | %d | %d | %d | %.3f | %d |\n", mode, N, peer, rounds, us / rounds, he + hb);
    fflush(stdout);
    return he;
  };
  printf("| mode | words | peer | rounds | us per round | errors |\n|---|---:|---:|---:|---:|---:|\n");
  run(0, 1024, 10, 0, true);
  run(3, 1, 2000, 1, false);   // another XCD
  run(3, 1, 2000, 8, false);   // the same XCD
  run(4, 1, 2000, 8, false);   // the same XCD, through L2
  for (int N : {64, 256, 512, 1024, 2048, 3072}) {
    run(0, N, 2000, 0, false);
    if (N >= ncu) run(9, N, 2000, 0, false);  // whole words per workgroup
  }
  for (int N : {256, 1024}) {
    run(5, N, 2000, 0, false);
    run(1, N, 2000, 0, false);
  }
  for (int N : {256, 1024}) run(12, N, 2000, 0, false);
  for (int N : {256, 512, 1024}) run(13, N, 2000, 0, false);
  return 0;
}
