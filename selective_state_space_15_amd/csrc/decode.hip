// Streaming decode of the mixer hot path on gfx950: new tokens stepped one at a time
// from the carried (h, conv buffer) state, for inference over streams longer than any
// one forward call (the two-million-token inference mode in the pith.science review
// of Video-Ma2mba, referee report summary).
//
// Per token t and head h (group g):
//   xin = the K-1 carried raw rows, then the new raw row xbc[t]
//   x, B, C = SiLU(bias + sum_k w[k] xin[k])  for the head's P x channels and the
//             group's N B and N C channels
//   dt = softplus(dt_raw + dt_bias), a = exp(dt A)
//   h[p][n] <- a h[p][n] + dt x[p] B[n];   y[p] = sum_n h[p][n] C[n] + D x[p]
//   out[p] = y[p] SiLU(z[p])
// which is the recurrence of the forward pass taken one step at a time.
//
// The rows p of a head's state are independent given B, C and dt, so one workgroup of
// 16 threads per row owns ROWS rows of one (batch, head): those rows of the fp32 state
// live in registers for the whole call (N / 16 elements per thread), each conv
// channel keeps its window of K-1 raw inputs in registers, and the post-conv x, B and C
// of the current token pass through LDS.  The state is read once and written once per
// call, whatever the number of tokens.  The B / C conv runs in every workgroup of the
// group (a few hundred channels); the group's first workgroup writes their carried rows.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace {

// 16 lanes per state row; ROWS state rows (head channels p) per workgroup: 16 (P/16
// workgroups per head) for few (batch, head) pairs, all P (one workgroup per head, 16 P
// threads) when there are enough heads to fill the GPU, which repeats the B / C conv
// P/16 times less
constexpr int kRowLanes = 16;

struct DecodeArgs {
  Problem pr;          // L = tokens in this call; h0 = state in (null = zeros)
  float* h_out;        // [B][H][P][N] (may equal h0)
  MView out;           // [B][T][H*P]
  MView cs_out;        // [B][K-1][Cd] conv state out (distinct from cs_in)
};

template <int NT>
__device__ __forceinline__ float sum_lanes(float v) {
  static_assert(NT == 4 || NT == 8 || NT == 16, "lanes per state row");
  if constexpr (NT == 16) return row_sum16(v);
  v += dpp_f<kDppQuad1032>(0.f, v);
  v += dpp_f<kDppQuad2301>(0.f, v);
  if constexpr (NT == 8) v += dpp_f<kDppRowHalfMirror>(0.f, v);
  return v;
}

template <typename IO, int P, int N, int K, int ROWS>
__global__ void __launch_bounds__(kRowLanes * ROWS) decode_kernel(DecodeArgs a) {
  constexpr int kDecThreads = kRowLanes * ROWS;
  constexpr int kRows = ROWS;
  using E = typename io_traits<IO>::elem;
  constexpr int SPLIT = P / kRows;      // workgroups per (batch, head)
  constexpr int NT = kDecThreads / kRows;  // threads per state row p
  constexpr int NPT = N / NT;           // state elements per thread
  constexpr int NCH = kRows + 2 * N;    // conv channels of one workgroup: its x rows, B, C
  constexpr int CPT = (NCH + kDecThreads - 1) / kDecThreads;  // channels per thread
  constexpr int KW = K > 1 ? K - 1 : 1;  // carried window
  static_assert(NT * kRows == kDecThreads && NPT * NT == N && SPLIT * kRows == P, "thread layout");
  const Problem& pr = a.pr;
  __shared__ float s_x[kRows], s_B[N], s_C[N];

  const int tid = threadIdx.x;
  const int part = blockIdx.x % SPLIT;
  const int b = blockIdx.x / (SPLIT * pr.H), h = (blockIdx.x / SPLIT) % pr.H;
  const int p0 = part * kRows;  // this workgroup's first state row
  const int hpg = pr.H / pr.G, g = h / hpg;
  const int64_t HP = static_cast<int64_t>(pr.H) * P;
  const int64_t GN = static_cast<int64_t>(pr.G) * N;

  // conv channels of this thread: list slot j = tid + 256 i; xbc channel ch[i]
  int64_t ch[CPT];
  bool live[CPT];
  float win[CPT][KW], wk[CPT][K > 0 ? K : 1], bias[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int j = tid + kDecThreads * i;
    live[i] = j < NCH;
    const int jj = live[i] ? j : 0;
    ch[i] = jj < kRows ? h * P + p0 + jj
                       : jj < kRows + N ? HP + g * N + (jj - kRows) : HP + GN + g * N + (jj - kRows - N);
    if constexpr (K > 0) {
#pragma unroll
      for (int k = 0; k < K; ++k) wk[i][k] = pr.conv_w[ch[i] * K + k];
      bias[i] = pr.conv_b ? pr.conv_b[ch[i]] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < KW; ++k) {
      float v = 0.f;
      if (K > 1 && pr.cs_in.p)
        v = io_traits<IO>::to_f(static_cast<const E*>(pr.cs_in.p)[b * pr.cs_in.sb + k * pr.cs_in.st + ch[i]]);
      win[i][k] = v;
    }
  }

  // state row p0 + pl (pl = tid / NT), columns n0 .. n0 + NPT
  const int pl = tid / NT, p = p0 + pl, n0 = (tid % NT) * NPT;
  float st[NPT];
  const int64_t soff = ((static_cast<int64_t>(b) * pr.H + h) * P + p) * N + n0;
#pragma unroll
  for (int j = 0; j < NPT; ++j) st[j] = pr.h0 ? pr.h0[soff + j] : 0.f;
  const float A = pr.A[h], Dh = pr.D ? pr.D[h] : 0.f;
  const float dtb = pr.dt_bias ? pr.dt_bias[h] : 0.f;
  const E* xbc = static_cast<const E*>(pr.xbc.p);
  const E* dtp = static_cast<const E*>(pr.dt.p);
  const bool gate = pr.z.p != nullptr;
  // without a gate the (unused) z loads read this row's x channel, always valid
  const E* zsrc = gate ? static_cast<const E*>(pr.z.p) + b * pr.z.sb + h * P + p
                       : xbc + b * pr.xbc.sb + h * P + p;
  const int64_t zst = gate ? pr.z.st : pr.xbc.st;
  // A token's raw row, dt and z are loaded one token ahead, unconditionally (the last
  // token reloads itself): with the state loads above they are all in flight at once,
  // instead of dt and z each waiting a memory round trip after the conv.
  E rawn[CPT], dtn, zn;
  auto issue_tok = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) rawn[i] = xbc[b * pr.xbc.sb + t * pr.xbc.st + ch[i]];
    dtn = dtp[b * pr.dt.sb + t * pr.dt.st + h];
    zn = zsrc[t * zst];
  };
  issue_tok(0);

  for (int64_t t = 0; t < pr.L; ++t) {
    E rawc[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) rawc[i] = rawn[i];
    const E dtc = dtn, zc = zn;
    issue_tok(t + 1 < pr.L ? t + 1 : t);
    // post-conv x, B, C of token t
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if (!live[i]) continue;
      const float raw = io_traits<IO>::to_f(rawc[i]);
      float v = raw;
      if constexpr (K > 0) {
        float pre = bias[i] + wk[i][K - 1] * raw;
#pragma unroll
        for (int k = 0; k < K - 1; ++k) pre += wk[i][k] * win[i][k];
        v = siluf_(pre);
#pragma unroll
        for (int k = 0; k + 1 < K - 1; ++k) win[i][k] = win[i][k + 1];
        if constexpr (K > 1) win[i][K - 2] = raw;
      }
      const int j = tid + kDecThreads * i;
      if (j < kRows) s_x[j] = v;
      else if (j < kRows + N) s_B[j - kRows] = v;
      else s_C[j - kRows - N] = v;
    }
    __syncthreads();
    float dt = io_traits<IO>::to_f(dtc) + dtb;
    if (pr.softplus) dt = softplusf_(dt);
    const float decay = __expf(dt * A);
    const float dtx = dt * s_x[pl];
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      st[j] = decay * st[j] + dtx * s_B[n0 + j];
      acc += st[j] * s_C[n0 + j];
    }
    const float y = sum_lanes<NT>(acc) + Dh * s_x[pl];
    if (tid % NT == 0) {
      float o = y;
      if (gate) o *= siluf_(io_traits<IO>::to_f(zc));
      static_cast<E*>(a.out.p)[b * a.out.sb + t * a.out.st + h * P + p] = io_traits<IO>::from_f(o);
    }
    __syncthreads();  // the next token rewrites s_x / s_B / s_C
  }

#pragma unroll
  for (int j = 0; j < NPT; ++j) a.h_out[soff + j] = st[j];
  if (K > 1 && a.cs_out.p) {
    // the last K-1 conv inputs: the window now (carried rows first when T < K-1)
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int j = tid + kDecThreads * i;
      // B / C rows: the group's first workgroup
      if (!live[i] || (j >= kRows && (h % hpg != 0 || part != 0))) continue;
#pragma unroll
      for (int k = 0; k < KW; ++k)
        static_cast<E*>(a.cs_out.p)[b * a.cs_out.sb + k * a.cs_out.st + ch[i]] = io_traits<IO>::from_f(win[i][k]);
    }
  }
}

// One token (T = 1) for many (batch, head) pairs: a grid of resident workgroups, each
// taking whole heads in turn (head q, q + grid, ...).  A head's inputs -- its state
// rows, conv window, taps, raw row, dt and z -- are loaded while the head before it
// computes and stores, so the state stream does not stop between heads (a workgroup per
// head would stream in rounds, each waiting for its loads).  Thread tid owns state row
// tid / 16, columns 16-wide interleaved as in decode_kernel, and conv channel tid (the
// head's P x channels, then the group's B and C channels).
template <typename IO, int P, int N, int K>
__global__ void __launch_bounds__(kRowLanes * P) decode_step_kernel(DecodeArgs a) {
  constexpr int NTHR = kRowLanes * P;
  using E = typename io_traits<IO>::elem;
  constexpr int NT = kRowLanes, NPT = N / NT;
  constexpr int NCH = P + 2 * N;  // conv channels of a head: its x rows, B, C
  constexpr int KW = K > 1 ? K - 1 : 1;
  static_assert(NCH <= NTHR, "one conv channel per thread");
  const Problem& pr = a.pr;
  __shared__ float s_x[P], s_B[N], s_C[N];
  const int tid = threadIdx.x;
  const int pl = tid / NT, n0 = (tid % NT) * NPT;
  const bool live = tid < NCH;
  const int jj = live ? tid : 0;
  const int hpg = pr.H / pr.G;
  const int64_t HP = static_cast<int64_t>(pr.H) * P;
  const int64_t GN = static_cast<int64_t>(pr.G) * N;
  const int64_t nblk = static_cast<int64_t>(pr.B) * pr.H;
  const E* xbc = static_cast<const E*>(pr.xbc.p);
  const E* dtp = static_cast<const E*>(pr.dt.p);
  const E* csi = static_cast<const E*>(pr.cs_in.p);
  const bool gate = pr.z.p != nullptr;
  const bool has_cs = K > 1 && csi != nullptr;

  // one head's inputs (every load unconditional, from a valid address)
  struct In {
    float st[NPT];
    float wk[K > 0 ? K : 1], bias;
    E win[KW], raw, dt, z;
  };
  auto chan = [&](int b, int h) -> int64_t {
    const int g = h / hpg;
    return jj < P ? h * P + jj : jj < P + N ? HP + g * N + (jj - P) : HP + GN + g * N + (jj - P - N);
  };
  auto load = [&](int64_t q, In& in) __attribute__((always_inline)) {
    const int b = static_cast<int>(q / pr.H), h = static_cast<int>(q % pr.H);
    const int64_t soff = ((static_cast<int64_t>(b) * pr.H + h) * P + pl) * N + n0;
#pragma unroll
    for (int j = 0; j < NPT; ++j) in.st[j] = pr.h0 ? pr.h0[soff + j] : 0.f;
    const int64_t c = chan(b, h);
    if constexpr (K > 0) {
#pragma unroll
      for (int k = 0; k < K; ++k) in.wk[k] = pr.conv_w[c * K + k];
      in.bias = pr.conv_b ? pr.conv_b[c] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < KW; ++k) in.win[k] = has_cs ? csi[b * pr.cs_in.sb + k * pr.cs_in.st + c] : E{};
    in.raw = xbc[b * pr.xbc.sb + c];
    in.dt = dtp[b * pr.dt.sb + h];
    in.z = gate ? static_cast<const E*>(pr.z.p)[b * pr.z.sb + h * P + pl] : in.raw;
  };

  In nx;
  int64_t q = blockIdx.x;
  load(q < nblk ? q : 0, nx);
  for (; q < nblk; q += gridDim.x) {
    const In cur = nx;
    load(q + gridDim.x < nblk ? q + gridDim.x : q, nx);
    const int b = static_cast<int>(q / pr.H), h = static_cast<int>(q % pr.H);
    // post-conv x, B, C of the token
    const float raw = io_traits<IO>::to_f(cur.raw);
    float v = raw;
    if constexpr (K > 0) {
      float pre = cur.bias + cur.wk[K - 1] * raw;
#pragma unroll
      for (int k = 0; k < K - 1; ++k) pre += cur.wk[k] * io_traits<IO>::to_f(cur.win[k]);
      v = siluf_(pre);
    }
    if (live) {
      if (tid < P) s_x[tid] = v;
      else if (tid < P + N) s_B[tid - P] = v;
      else s_C[tid - P - N] = v;
    }
    __syncthreads();
    float dt = io_traits<IO>::to_f(cur.dt) + (pr.dt_bias ? pr.dt_bias[h] : 0.f);
    if (pr.softplus) dt = softplusf_(dt);
    const float decay = __expf(dt * pr.A[h]);
    const float xv = s_x[pl];
    const float dtx = dt * xv;
    float st[NPT], acc = 0.f;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      st[j] = decay * cur.st[j] + dtx * s_B[n0 + j];
      acc += st[j] * s_C[n0 + j];
    }
    const float y = sum_lanes<NT>(acc) + (pr.D ? pr.D[h] : 0.f) * xv;
    if (tid % NT == 0) {
      float o = y;
      if (gate) o *= siluf_(io_traits<IO>::to_f(cur.z));
      static_cast<E*>(a.out.p)[b * a.out.sb + h * P + pl] = io_traits<IO>::from_f(o);
    }
    const int64_t soff = ((static_cast<int64_t>(b) * pr.H + h) * P + pl) * N + n0;
#pragma unroll
    for (int j = 0; j < NPT; ++j) a.h_out[soff + j] = st[j];
    // the conv window after the token: the carried rows shifted by one, then the raw row;
    // B / C rows by the group's first head
    if (K > 1 && a.cs_out.p && live && (tid < P || h % hpg == 0)) {
      const int64_t c = chan(b, h);
#pragma unroll
      for (int k = 0; k < KW; ++k)
        static_cast<E*>(a.cs_out.p)[b * a.cs_out.sb + k * a.cs_out.st + c] = k + 1 < KW ? cur.win[k + 1] : cur.raw;
    }
    __syncthreads();  // the next head rewrites s_x / s_B / s_C
  }
}

template <typename IO, int P, int N, int ROWS>
hipError_t launch_decode_rows(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.pr.B * a.pr.H * (P / ROWS))), block(kRowLanes * ROWS);
  switch (a.pr.K) {
    case 0: hipLaunchKernelGGL((decode_kernel<IO, P, N, 0, ROWS>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<IO, P, N, 2, ROWS>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((decode_kernel<IO, P, N, 3, ROWS>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<IO, P, N, 4, ROWS>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename IO, int P, int N, int K>
hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t s) {
  const void* kf = reinterpret_cast<const void*>(&decode_step_kernel<IO, P, N, K>);
  const int64_t nblk = static_cast<int64_t>(a.pr.B) * a.pr.H;
  const int64_t res = resident_blocks(kf, kRowLanes * P);
  if (res <= 0) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nblk < res ? nblk : res)), block(kRowLanes * P);
  hipLaunchKernelGGL((decode_step_kernel<IO, P, N, K>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename IO, int P, int N>
hipError_t launch_decode_pn(const DecodeArgs& a, hipStream_t s) {
  // whole heads from 512 (batch, head) pairs on (two or more workgroups per CU); one
  // token there streams the heads through resident workgroups
  if (static_cast<int64_t>(a.pr.B) * a.pr.H >= 512) {
    if (a.pr.L == 1) {
      switch (a.pr.K) {
        case 0: return launch_decode_step<IO, P, N, 0>(a, s);
        case 2: return launch_decode_step<IO, P, N, 2>(a, s);
        case 3: return launch_decode_step<IO, P, N, 3>(a, s);
        case 4: return launch_decode_step<IO, P, N, 4>(a, s);
        default: return hipErrorInvalidValue;
      }
    }
    return launch_decode_rows<IO, P, N, P>(a, s);
  }
  return launch_decode_rows<IO, P, N, 16>(a, s);
}

template <typename IO>
hipError_t launch_decode_io(const DecodeArgs& a, hipStream_t s) {
#define SSD_DEC(PP, NN) \
  if (a.pr.P == PP && a.pr.N == NN) return launch_decode_pn<IO, PP, NN>(a, s);
  SSD_DEC(64, 128)
  SSD_DEC(64, 64)
  SSD_DEC(64, 32)
  SSD_DEC(64, 16)
  SSD_DEC(32, 128)
  SSD_DEC(32, 64)
  SSD_DEC(32, 32)
  SSD_DEC(32, 16)
#undef SSD_DEC
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const Problem& pr, float* h_out, MView out, MView cs_out, hipStream_t s) {
  DecodeArgs a{pr, h_out, out, cs_out};
  TimingScope ts(kKDecode, s);
  return pr.bf16 ? launch_decode_io<bf16_t>(a, s) : launch_decode_io<float>(a, s);
}

}  // namespace ssd
