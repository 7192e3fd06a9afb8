// Chunk loaders shared by the forward and backward kernels.
//
// conv_rows: the post-conv rows [t0, t0+64) of the x (head h), B and C (group g)
//   channel segments.  For x with conv width K > 0 the raw rows t0-3 .. t0+63 are
//   read (rows < 0 from the carried conv state, rows >= L as zero) and
//       pre[t,c] = bias[c] + sum_{k<K} w[c,k] * xin[t-K+1+k, c],  value = silu(pre)
//   is evaluated in registers (the causal depthwise conv of the Video-Ma2mba
//   review's Conv1d critique, skeptic critique of the pith.science verdict).
//   B and C are shared by every head of a group, so their conv runs once in a
//   pre-pass (Problem::bc); here they are only loaded.  The backward, which reads
//   the x rows of a chunk in two kernels, also takes x from a pre-pass
//   (Problem::xp), computed with the same arithmetic, so the values are identical.
//   Without conv all rows are passed through.  Rows >= L are delivered as zero.
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
          int RB = 8, bool XPRE = true>  // XPRE: may take x from Problem::xp
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
  // issue_raw(): which loaded vectors are live (bit q (RX + 3) + i for x, then
  // XT (RX + 3) + q RB + r for B / C); the others are zeroed when consumed
  static constexpr int kXBits = DX ? XT * (RX + 3) : 0;
  static_assert(kXBits + (DB || DC ? BT * RB : 0) <= 32, "mask bits fit one word");
  uint32_t okm = 0;

  // Branch-free form of issue(): every load reads a valid row (clamped into the
  // sequence, or the carried conv state), nothing here uses the loaded values, and
  // the masks are kept as bits for consume_raw_lds_taps().  Issued a chunk ahead, the
  // loads stay in flight until the consuming chunk: a branch around a load, or a
  // select right after it, would make the wave wait for it at once.
  __device__ __forceinline__ void issue_raw(const Problem& pr, int b, int h, int g, int64_t t0) {
    const int K = pr.K;
    uint32_t m = 0;
    if constexpr (DX) {
      const bool pre = XPRE && pr.xp.p != nullptr;  // post-conv rows: slots 3 ..
      const E* base = pre ? static_cast<const E*>(pr.xp.p) + b * pr.xp.sb
                          : static_cast<const E*>(pr.xbc.p) + b * pr.xbc.sb;
      const int64_t st = pre ? pr.xp.st : pr.xbc.st;
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
          const bool live = task < NTX && !((K == 0 || pre) && i < 3) && t < pr.L;
          const bool from_state = t < 0 && !pre && csi && t >= -(K - 1);
          const bool ok = live && (t >= 0 || from_state);
          const int64_t tc = t < 0 ? 0 : (t < pr.L ? t : pr.L - 1);
          const E* src = from_state ? csi + (t + K - 1) * pr.cs_in.st + c : base + tc * st + c;
          xin[q][i] = *reinterpret_cast<const uint4*>(src);
          m |= (ok ? 1u : 0u) << (q * (RX + 3) + i);
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
          const bool ok = task < NTB && t < pr.L;
          bin[q][r] = *reinterpret_cast<const uint4*>(col + (t < pr.L ? t : pr.L - 1) * sst);
          m |= (ok ? 1u : 0u) << (kXBits + q * RB + r);
        }
      }
    }
    okm = m;
  }

  __device__ __forceinline__ void issue(const Problem& pr, int b, int h, int g, int64_t t0) {
    // interior chunk: every row it touches (conv halo included) is inside the
    // sequence, so the loads need no masks and the rows are plain stride steps
    constexpr bool XFULL = NTX % NTHR == 0, BFULL = NTB % NTHR == 0;
    if (t0 >= 3 && t0 + kQ <= pr.L) {
      if constexpr (DX) {
        const bool pre = XPRE && pr.xp.p != nullptr;
        const E* base = pre ? static_cast<const E*>(pr.xp.p) + b * pr.xp.sb
                            : static_cast<const E*>(pr.xbc.p) + b * pr.xbc.sb;
        const int64_t st = pre ? pr.xp.st : pr.xbc.st;
        const int first = pre ? 3 : 0;  // post-conv rows skip the halo slots
#pragma unroll
        for (int q = 0; q < XT; ++q) {
          const int task = threadIdx.x + q * NTHR;
          if (!XFULL && task >= NTX) continue;
          const int cl = (task % (P / V)) * V;
          const int r0 = (task / (P / V)) * RX;
          const E* rowp = base + (t0 + r0 - 3) * st + h * P + cl;
#pragma unroll
          for (int i = 0; i < RX + 3; ++i)
            if (i >= first) xin[q][i] = *reinterpret_cast<const uint4*>(rowp + i * st);
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
          if (!BFULL && task >= NTB) continue;
          const int grp = task % (GB + GC);
          const int r0 = (task / (GB + GC)) * RB;
          const bool isB = grp < GB;
          const E* rowp = src + (isB ? cB + grp * V : cC + (grp - GB) * V) + (t0 + r0) * sst;
#pragma unroll
          for (int r = 0; r < RB; ++r) bin[q][r] = *reinterpret_cast<const uint4*>(rowp + r * sst);
        }
      }
      return;
    }
    const int K = pr.K;
    if constexpr (DX) {
      const E* xbc = static_cast<const E*>(pr.xbc.p) + b * pr.xbc.sb;
      const E* csi = pr.cs_in.p ? static_cast<const E*>(pr.cs_in.p) + b * pr.cs_in.sb : nullptr;
      if (XPRE && pr.xp.p) {
        // post-conv rows from the pre-pass: rows t0 + r0 .. + RX - 1 into slots 3 ..
        const E* xp = static_cast<const E*>(pr.xp.p) + b * pr.xp.sb;
#pragma unroll
        for (int q = 0; q < XT; ++q) {
          const int task = threadIdx.x + q * NTHR;
          const int cl = (task % (P / V)) * V;
          const int r0 = (task / (P / V)) * RX;
#pragma unroll
          for (int i = 0; i < RX; ++i) {
            const bool ok = task < NTX && t0 + r0 + i < pr.L;
            const int64_t t = ok ? t0 + r0 + i : t0;  // masked rows read a valid row
            xin[q][3 + i] = keep_if(ok, *reinterpret_cast<const uint4*>(xp + t * pr.xp.st + h * P + cl));
          }
        }
      } else
#pragma unroll
      for (int q = 0; q < XT; ++q) {
        const int task = threadIdx.x + q * NTHR;
        const int cl = (task % (P / V)) * V;
        const int r0 = (task / (P / V)) * RX;
        const int c = h * P + cl;
#pragma unroll
        for (int i = 0; i < RX + 3; ++i) {
          // every load is unconditional: masked rows read row t0 of xbc (always valid)
          const int64_t t = t0 + r0 - 3 + i;
          const bool live = task < NTX && !(K == 0 && i < 3) && t < pr.L;
          const bool from_state = t < 0;
          const bool ok = live && (!from_state || (csi && t >= -(K - 1)));
          const E* src = xbc + t0 * pr.xbc.st + c;
          if (ok) src = from_state ? csi + (t + K - 1) * pr.cs_in.st + c : xbc + t * pr.xbc.st + c;
          xin[q][i] = keep_if(ok, *reinterpret_cast<const uint4*>(src));
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
          const bool ok = task < NTB && t0 + r0 + r < pr.L;
          const int64_t t = ok ? t0 + r0 + r : t0;  // masked rows read a valid row
          bin[q][r] = keep_if(ok, *reinterpret_cast<const uint4*>(col + t * sst));
        }
      }
    }
  }

  template <typename F>
  __device__ __forceinline__ void consume(const Problem& pr, int h, int64_t t0, F&& put) const {
    consume_impl<false>(pr, h, t0, put, nullptr);
  }
  // wl: LDS copy of the head's conv taps and bias, [P][5] (taps right-aligned on 4,
  // bias last), so a chunk loop does not re-read them from global memory.
  template <typename F>
  __device__ __forceinline__ void consume_lds_taps(const Problem& pr, int h, int64_t t0, F&& put,
                                                   const float* wl) const {
    consume_impl<true>(pr, h, t0, put, wl);
  }
  // after issue_raw(): the masks are applied here
  template <typename F>
  __device__ __forceinline__ void consume_raw_lds_taps(const Problem& pr, int h, int64_t t0, F&& put,
                                                       const float* wl) const {
    consume_impl<true, true>(pr, h, t0, put, wl);
  }

  // The B / C rows of issue_raw() as the loaded 16-byte vectors (zero where masked),
  // for tiles that keep the I/O element type: put_raw(seg, row, local_channel, uint4).
  // No conversion round trip through fp32.
  template <typename F>
  __device__ __forceinline__ void consume_bc_raw(F&& put_raw) const {
    static_assert(DB || DC, "B / C rows only");
#pragma unroll
    for (int q = 0; q < BT; ++q) {
      const int task = threadIdx.x + q * NTHR;
      if (NTB % NTHR != 0 && task >= NTB) continue;
      const int grp = task % (GB + GC);
      const int r0 = (task / (GB + GC)) * RB;
      const int seg = grp < GB ? 1 : 2;
      const int cl = (seg == 1 ? grp : grp - GB) * V;
#pragma unroll
      for (int r = 0; r < RB; ++r) put_raw(seg, r0 + r, cl, keep_if((okm >> (kXBits + q * RB + r)) & 1u, bin[q][r]));
    }
  }

  template <bool WLDS, bool RAW = false, typename F>
  __device__ __forceinline__ void consume_impl(const Problem& pr, int h, int64_t t0, F&& put,
                                               const float* wl) const {
    auto xv = [&](int q, int i) -> uint4 {
      if constexpr (RAW) return keep_if((okm >> (q * (RX + 3) + i)) & 1u, xin[q][i]);
      else return xin[q][i];
    };
    auto bv = [&](int q, int r) -> uint4 {
      if constexpr (RAW) return keep_if((okm >> (kXBits + q * RB + r)) & 1u, bin[q][r]);
      else return bin[q][r];
    };
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
        if (K > 0 && !(XPRE && pr.xp.p)) {
          if constexpr (WLDS) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
              const float* wv = wl + (cl + v) * 5;
#pragma unroll
              for (int j = 0; j < 4; ++j) w4[j][v] = wv[j];
              bias[v] = wv[4];
            }
          } else {
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
        }
#pragma unroll
        for (int r = 0; r < RX; ++r) {
          float o[V];
          if (K > 0 && !(XPRE && pr.xp.p)) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
              float pre = bias[v];
#pragma unroll
              for (int j = 0; j < 4; ++j) pre = fmaf(w4[j][v], raw_elem<IO>(xv(q, r + j), v), pre);
              o[v] = siluf_(pre);
            }
          } else {
#pragma unroll
            for (int v = 0; v < V; ++v) o[v] = raw_elem<IO>(xv(q, r + 3), v);
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
          for (int v = 0; v < V; ++v) o[v] = raw_elem<IO>(bv(q, r), v);
          put(seg, r0 + r, cl, o);
        }
      }
    }
  }
};

// One-shot form of ChunkLoader (issue then consume).
template <typename IO, int P, int N, bool DX, bool DB, bool DC, int NTHR = kThreads, typename F>
__device__ __forceinline__ void conv_rows(const Problem& pr, int b, int h, int g, int64_t t0,
                                          F&& put) {
  ChunkLoader<IO, P, N, DX, DB, DC, NTHR> ld;
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

// Four consecutive LDS operand elements from floats: 8 bytes (bf16) or 16 (fp32).
template <typename IO>
__device__ __forceinline__ void lds_put4(typename io_traits<IO>::lds* dst, float a, float b, float c, float d) {
  if constexpr (sizeof(typename io_traits<IO>::lds) == 2)
    *reinterpret_cast<uint2*>(dst) = make_uint2(f2bf2(a, b), f2bf2(c, d));
  else
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}

// Store 16 bytes worth of floats into an LDS row as I/O-typed operand elements.
template <typename IO>
__device__ __forceinline__ void lds_put_row(typename io_traits<IO>::lds* dst, const float* v) {
  store_vec16<IO>(reinterpret_cast<typename io_traits<IO>::elem*>(dst), v);
}

}  // namespace ssd
