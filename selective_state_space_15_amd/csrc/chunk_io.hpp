// Chunk loaders shared by the forward and backward kernels.
//
// conv_rows: the post-conv rows [t0, t0+64) of the x (head h), B and C (group g)
//   channel segments.  For x with conv width K > 0 the raw rows t0-3 .. t0+63 are
//   read (rows < 0 from the carried conv state, rows >= L as zero) and
//       pre[t,c] = bias[c] + sum_{k<K} w[c,k] * xin[t-K+1+k, c],  value = silu(pre)
//   is evaluated in registers (the causal depthwise conv of the Video-Ma2mba
//   review's Conv1d critique, skeptic critique of the pith.science verdict).
//   B and C are shared by every head of a group, so their conv runs once in a
//   pre-pass (Problem::bc); here they are only loaded.  Without conv all rows are
//   passed through.  Rows >= L are delivered as zero.
//   Each delivered row vector (16 bytes of I/O elements, as floats) goes to
//   put(seg, row, local_channel, const float* v) with seg 0 = x, 1 = B, 2 = C.
//
// plain_rows: rows [t0, t0+64) of one [B, L, *] view, W channels from col0
//   (no conv), delivered the same way (seg = 0); rows >= L are zero.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace ssd {

// Two-phase chunk loader: issue() starts the global loads of one chunk into
// registers (so they can be in flight while the previous chunk computes);
// consume() turns them into post-conv rows and hands them to put().
template <typename IO, int P, int N, bool DX, bool DB, bool DC, int NTHR = kThreads, int RX = 2,
          int RB = 8>
struct ChunkLoader {
  using T = io_traits<IO>;
  using E = typename T::elem;
  static constexpr int V = T::vec;
  static constexpr int NTX = DX ? (P / V) * (kQ / RX) : 0;       // x tasks (RX rows each)
  static constexpr int XT = (NTX + NTHR - 1) / NTHR;             // x tasks per thread
  static constexpr int GB = DB ? N / V : 0, GC = DC ? N / V : 0;
  static constexpr int NTB = (GB + GC) * (kQ / RB);              // B/C tasks (RB rows each)
  static constexpr int BT = (NTB + NTHR - 1) / NTHR;             // B/C tasks per thread
  uint4 xin[XT > 0 ? XT : 1][RX + 3];
  uint4 bin[BT > 0 ? BT : 1][RB];

  __device__ __forceinline__ void issue(const Problem& pr, int b, int h, int g, int64_t t0) {
    const int K = pr.K;
    if constexpr (DX) {
      const E* xbc = static_cast<const E*>(pr.xbc.p) + b * pr.xbc.sb;
      const E* csi = pr.cs_in.p ? static_cast<const E*>(pr.cs_in.p) + b * pr.cs_in.sb : nullptr;
#pragma unroll
      for (int q = 0; q < XT; ++q) {
        const int task = threadIdx.x + q * NTHR;
        const int cl = (task % (P / V)) * V;
        const int r0 = (task / (P / V)) * RX;
        const int c = h * P + cl;
#pragma unroll
        for (int i = 0; i < RX + 3; ++i) {
          const int64_t t = t0 + r0 - 3 + i;
          xin[q][i] = make_uint4(0u, 0u, 0u, 0u);
          if (task >= NTX || (K == 0 && i < 3) || t >= pr.L) {
          } else if (t >= 0) {
            xin[q][i] = *reinterpret_cast<const uint4*>(xbc + t * pr.xbc.st + c);
          } else if (csi && t >= -(K - 1)) {
            xin[q][i] = *reinterpret_cast<const uint4*>(csi + (t + K - 1) * pr.cs_in.st + c);
          }
        }
      }
    }
    if constexpr (DB || DC) {
      const bool pre = pr.bc.p != nullptr;
      const E* src = pre ? static_cast<const E*>(pr.bc.p) + b * pr.bc.sb
                         : static_cast<const E*>(pr.xbc.p) + b * pr.xbc.sb;
      const int64_t sst = pre ? pr.bc.st : pr.xbc.st;
      const int cB = (pre ? 0 : pr.H * P) + g * N;
      const int cC = (pre ? 0 : pr.H * P) + pr.G * N + g * N;
#pragma unroll
      for (int q = 0; q < BT; ++q) {
        const int task = threadIdx.x + q * NTHR;
        const int grp = task % (GB + GC);
        const int r0 = (task / (GB + GC)) * RB;
        const bool isB = grp < GB;
        const E* col = src + (isB ? cB + grp * V : cC + (grp - GB) * V);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const int64_t t = t0 + r0 + r;
          bin[q][r] = (task < NTB && t < pr.L) ? *reinterpret_cast<const uint4*>(col + t * sst)
                                               : make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
  }

  template <typename F>
  __device__ __forceinline__ void consume(const Problem& pr, int h, int64_t t0, F&& put) const {
    const int K = pr.K;
    if constexpr (DX) {
#pragma unroll
      for (int q = 0; q < XT; ++q) {
        const int task = threadIdx.x + q * NTHR;
        if (task >= NTX) continue;
        const int cl = (task % (P / V)) * V;
        const int r0 = (task / (P / V)) * RX;
        const int c = h * P + cl;
        float w4[4][V], bias[V];
        if (K > 0) {
#pragma unroll
          for (int v = 0; v < V; ++v) {
            bias[v] = pr.conv_b ? pr.conv_b[c + v] : 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int kk = j - (4 - K);  // taps right-aligned on 4
              w4[j][v] = kk >= 0 ? pr.conv_w[(c + v) * K + kk] : 0.f;
            }
          }
        }
#pragma unroll
        for (int r = 0; r < RX; ++r) {
          float o[V];
          if (K > 0) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
              float pre = bias[v];
#pragma unroll
              for (int j = 0; j < 4; ++j) pre = fmaf(w4[j][v], raw_elem<IO>(xin[q][r + j], v), pre);
              o[v] = siluf_(pre);
            }
          } else {
#pragma unroll
            for (int v = 0; v < V; ++v) o[v] = raw_elem<IO>(xin[q][r + 3], v);
          }
          if (t0 + r0 + r >= pr.L)
#pragma unroll
            for (int v = 0; v < V; ++v) o[v] = 0.f;
          put(0, r0 + r, cl, o);
        }
      }
    }
    if constexpr (DB || DC) {
#pragma unroll
      for (int q = 0; q < BT; ++q) {
        const int task = threadIdx.x + q * NTHR;
        if (task >= NTB) continue;
        const int grp = task % (GB + GC);
        const int r0 = (task / (GB + GC)) * RB;
        const int seg = grp < GB ? 1 : 2;
        const int cl = (seg == 1 ? grp : grp - GB) * V;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          float o[V];
#pragma unroll
          for (int v = 0; v < V; ++v) o[v] = raw_elem<IO>(bin[q][r], v);
          put(seg, r0 + r, cl, o);
        }
      }
    }
  }
};

// One-shot form of ChunkLoader (issue then consume).
template <typename IO, int P, int N, bool DX, bool DB, bool DC, typename F>
__device__ __forceinline__ void conv_rows(const Problem& pr, int b, int h, int g, int64_t t0,
                                          F&& put) {
  ChunkLoader<IO, P, N, DX, DB, DC> ld;
  ld.issue(pr, b, h, g, t0);
  ld.consume(pr, h, t0, put);
}

template <typename IO, int W, typename F>
__device__ __forceinline__ void plain_rows(const View& vw, int64_t L, int b, int col0, int64_t t0,
                                           F&& put) {
  using T = io_traits<IO>;
  using E = typename T::elem;
  constexpr int V = T::vec;
  constexpr int NG = W / V;
  const E* base = static_cast<const E*>(vw.p) + b * vw.sb + col0;
  for (int task = threadIdx.x; task < NG * kQ; task += kThreads) {
    const int grp = task % NG;
    const int r = task / NG;
    const int64_t t = t0 + r;
    vec16<IO> v;
    if (t < L)
      load_vec16<IO>(v, base + t * vw.st + grp * V);
    else
      zero_vec16<IO>(v);
    put(0, r, grp * V, v.v);
  }
}

// Store 16 bytes worth of floats into an LDS row as I/O-typed operand elements.
template <typename IO>
__device__ __forceinline__ void lds_put_row(typename io_traits<IO>::lds* dst, const float* v) {
  store_vec16<IO>(reinterpret_cast<typename io_traits<IO>::elem*>(dst), v);
}

}  // namespace ssd
