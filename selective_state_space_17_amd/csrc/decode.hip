// Token-by-token state update ("decode") for gfx950 (MI355X).
//
// At inference a state space layer keeps only its state and advances it one
// token at a time at a cost that does not depend on how many tokens came
// before ("03 - Modelos de espacio de estados", "Coste de inferencia"; the
// fixed-size state of "P20 - Mamba", 5).  These kernels apply the same
// recurrence and readout as the sequence kernels to T >= 1 new tokens,
// reading the state from HBM and writing it back in place:
//   Mamba-1, per (b, c, n):  h <- exp(delta A[c,n]) h + delta B[n] x
//                            y = sum_n C[n] h + D[c] x,  out = y * silu(z)
//   Mamba-2 multi-head, per (b, h, p, n) with scalar A[h] and group g(h):
//                            S <- exp(delta A[h]) S + delta B[g,n] x[p]
//                            y[p] = sum_n C[g,n] S + D[h] x[p],  out = y * silu(z)
//   Mamba-3 SISO rule (TRAP; "Mamba-3" blog, "El modelo Mamba-3" item 1), with a = exp(delta A[h]):
//                            S <- a S + (1 - lam) delta a B_prev[g,n] x_prev[p] + lam delta B[g,n] x[p]
//   where x_prev, B_prev are the previous token's (given for the first new token; zero if absent).
//   Complex-valued state (ROT; "El modelo Mamba-3" item 2, rotations per "Arquitectura"): each state
//   pair (2k, 2k+1) is one complex number and the transition exp(delta (A[h] + i omega[h,k])) also
//   rotates it by delta*omega: (u, v) <- (c u - s v, s u + c v), c, s = cos, sin(delta*omega).
// The work per token is a few operations per byte of state, so the kernels
// are bound by HBM: one thread owns 4 consecutive states of one row (one
// 16-byte load and store when the layout allows), a row's threads are
// consecutive lanes, and the readout's sum over states is a butterfly over
// those lanes.  Consecutive threads touch consecutive 16-byte pieces of the
// state, so every access to it is fully coalesced.
#include <type_traits>

#include "internal.h"

namespace mssm {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kThreads = 256;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));   // round to nearest even
}
__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + exp2_hw(-z * kLog2e)); }

// sine and cosine of an angle in radians: reduce it to revolutions in [-1/2, 1/2] (the fp32 product
// is off by at most |angle| * 2^-24 revolutions), then the hardware's sine and cosine, which take
// their argument in revolutions.  An angle of 0 gives exactly 0 and 1.
__device__ __forceinline__ void sincos_rev(float angle, float& s, float& c) {
  const float rev = angle * 0.159154943091895336f;   // 1 / (2 pi)
  const float r = rev - __builtin_rintf(rev);
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
}

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// sum over the lpr lanes of an aligned group (lpr a power of two <= 64; uniform):
// quad swaps, then half-row and row mirrors, then cross-row shuffles
__device__ __forceinline__ float group_sum(float v, int lpr) {
  if (lpr >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if (lpr >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if (lpr >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if (lpr >= 16) v += dpp<0x140>(v);  // row_mirror
  if (lpr >= 32) v += __shfl_xor(v, 16, 64);
  if (lpr >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// S (4 or 8) states n0..n0+S-1 of a row (entries past N read as 0 and are not written).
// The state is touched once per token: its vector accesses carry the
// non-temporal (streaming) cache hint, which measured 3-17 % faster.
using f32v4 = float __attribute__((ext_vector_type(4)));
template <int S, bool VEC>
__device__ __forceinline__ void loadS(const float* p, int n0, int N, float (&v)[S]) {
  if constexpr (VEC) {   // N % S == 0: a group is wholly inside or wholly past the row
#pragma unroll
    for (int i = 0; i < S / 4; ++i) {
      const float4 t = n0 < N ? __builtin_bit_cast(float4, __builtin_nontemporal_load(
                                    reinterpret_cast<const f32v4*>(p + n0 + 4 * i)))
                              : float4{0.f, 0.f, 0.f, 0.f};
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < S; ++q) v[q] = n0 + q < N ? p[n0 + q] : 0.f;
  }
}
template <int S, bool VEC>
__device__ __forceinline__ void storeS(float* p, int n0, int N, const float (&v)[S]) {
  if constexpr (VEC) {
    if (n0 < N) {
#pragma unroll
      for (int i = 0; i < S / 4; ++i)
        __builtin_nontemporal_store(f32v4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]},
                                    reinterpret_cast<f32v4*>(p + n0 + 4 * i));
    }
  } else {
#pragma unroll
    for (int q = 0; q < S; ++q)
      if (n0 + q < N) p[n0 + q] = v[q];
  }
}
// S consecutive B or C values (8- or 16-byte loads when N % S == 0)
template <typename T, int S, bool VEC>
__device__ __forceinline__ void loadSio(const T* p, int n0, int N, float (&v)[S]) {
  if constexpr (VEC) {
    if (n0 < N) {
#pragma unroll
      for (int i = 0; i < S / 4; ++i) {
        if constexpr (sizeof(T) == 2) {
          const uint2 w = *reinterpret_cast<const uint2*>(p + n0 + 4 * i);
          v[4 * i] = __uint_as_float(w.x << 16); v[4 * i + 1] = __uint_as_float(w.x & 0xffff0000u);
          v[4 * i + 2] = __uint_as_float(w.y << 16); v[4 * i + 3] = __uint_as_float(w.y & 0xffff0000u);
        } else {
          const float4 w = *reinterpret_cast<const float4*>(p + n0 + 4 * i);
          v[4 * i] = w.x; v[4 * i + 1] = w.y; v[4 * i + 2] = w.z; v[4 * i + 3] = w.w;
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < S; ++q) v[q] = 0.f;
    }
  } else {
#pragma unroll
    for (int q = 0; q < S; ++q) v[q] = n0 + q < N ? to_f32(p[n0 + q]) : 0.f;
  }
}

struct UpdParams {
  float* state;
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  void* out;
  int64_t batch, L, N;
  int64_t dim;             // Mamba-1: channels
  int64_t H, P, G;         // multi-head form
  int64_t rows;            // rows of the state
  int lpr;                 // lanes per row
  // Mamba-1 with the short causal convolution in front (x is then its input)
  const float* conv_w;     // [dim, conv_width]
  const float* conv_b;     // [dim], nullable
  const void* conv_in;     // [batch, conv_width - 1, dim] (io dtype): the window before the first
                           // token (nullable: zero inputs)
  void* conv_out;          // the window after the last token (nullable: not written); both are
                           // conv_state for a decode step, conv_init and nothing for a sequence
  int conv_width;
  // multi-head form with the Mamba-3 exponential-trapezoidal rule (TRAP)
  const void* lam;         // [batch, L, H]
  const void* x_prev;      // [batch, H, P], nullable
  const void* B_prev;      // [batch, G, N], nullable
  const float* omega;      // [H, N/2] (ROT)
  int64_t rank;            // MIMO: inputs and outputs per channel (x, z, out [batch, L, H, rank, P],
                           // B, C [batch, L, G, rank, N]; x_prev [batch, H, rank, P], B_prev [batch, G, rank, N])
  // the state read before the first token (nullable: zero) and written after
  // the last (nullable: not written); both are `state` for an update in place,
  // h0 and final_state for a whole sequence
  const float* state_in;
  float* state_out;
};

// Each thread owns S states (4, or 8 when dstate allows: two 16-byte loads
// in flight per lane) in each of R rows spaced a grid-width of rows apart (so
// every pass over r is one coalesced sweep).  One row per thread measured
// fastest: it keeps registers low enough for 8 waves per SIMD.
constexpr int R = 1;

// Mamba-1: row = (b, c), state [batch, dim, N]
template <typename T, bool VEC, int S, bool CONV>
__global__ __launch_bounds__(kThreads) void scan_update_kernel(UpdParams p) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t row0 = gid / p.lpr;
  const int64_t rstride = static_cast<int64_t>(gridDim.x) * kThreads / p.lpr;
  const int n0 = S * static_cast<int>(gid % p.lpr);
  const int N = static_cast<int>(p.N);
  const int64_t L = p.L, dim = p.dim;
  const T* x = static_cast<const T*>(p.x);
  const T* delta = static_cast<const T*>(p.delta);
  const T* Bm = static_cast<const T*>(p.B);
  const T* Cm = static_cast<const T*>(p.C);
  const T* z = static_cast<const T*>(p.z);
  T* out = static_cast<T*>(p.out);

  bool live[R];
  int64_t rr[R], bb[R], cc[R];
  float h[R][S], a2[R][S], Dc[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t row = row0 + k * rstride;
    live[k] = row < p.rows;
    rr[k] = live[k] ? row : 0;
    bb[k] = rr[k] / dim;
    cc[k] = rr[k] % dim;
    if (p.state_in != nullptr) {
      loadS<S, VEC>(p.state_in + rr[k] * N, n0, N, h[k]);
    } else {
#pragma unroll
      for (int q = 0; q < S; ++q) h[k][q] = 0.f;
    }
    loadS<S, VEC>(p.A + cc[k] * N, n0, N, a2[k]);
    Dc[k] = p.D != nullptr ? p.D[cc[k]] : 0.f;
  }
  // convolution (CONV): taps right-aligned into 4 slots (slot 3 = this token),
  // win[j] = the input 3 - j tokens back, taken from conv_in and returned to conv_out
  float cw[R][4], cbias[R], win[R][3];
  if constexpr (CONV) {
    const int W = p.conv_width;
    const T* cs = static_cast<const T*>(p.conv_in);
#pragma unroll
    for (int k = 0; k < R; ++k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) cw[k][j] = j >= 4 - W ? p.conv_w[cc[k] * W + (j - (4 - W))] : 0.f;
      cbias[k] = p.conv_b != nullptr ? p.conv_b[cc[k]] : 0.f;
#pragma unroll
      for (int m = 1; m <= 3; ++m)
        win[k][3 - m] = (m <= W - 1 && cs != nullptr) ? to_f32(cs[(bb[k] * (W - 1) + (W - 1 - m)) * dim + cc[k]]) : 0.f;
    }
  }
  for (int64_t t = 0; t < L; ++t) {
    float d[R], u[R], zz[R], bv[R][S], cv[R][S];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int64_t o = (bb[k] * L + t) * dim + cc[k];
      d[k] = to_f32(delta[o]);
      u[k] = to_f32(x[o]);
      if constexpr (CONV) {
        const float xin = u[k];
        float a = __builtin_fmaf(cw[k][3], xin, cbias[k]);
        a = __builtin_fmaf(cw[k][2], win[k][2], a);
        a = __builtin_fmaf(cw[k][1], win[k][1], a);
        a = __builtin_fmaf(cw[k][0], win[k][0], a);
        u[k] = silu(a);
        win[k][0] = win[k][1];
        win[k][1] = win[k][2];
        win[k][2] = xin;
      }
      zz[k] = z != nullptr ? to_f32(z[o]) : 0.f;
      loadSio<T, S, VEC>(Bm + (bb[k] * L + t) * N, n0, N, bv[k]);
      loadSio<T, S, VEC>(Cm + (bb[k] * L + t) * N, n0, N, cv[k]);
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float du = d[k] * u[k];
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < S; ++q) {
        h[k][q] = __builtin_fmaf(exp2_hw(d[k] * a2[k][q] * kLog2e), h[k][q], du * bv[k][q]);
        acc = __builtin_fmaf(cv[k][q], h[k][q], acc);
      }
      acc = group_sum(acc, p.lpr);
      if (live[k] && n0 == 0) {
        float y = __builtin_fmaf(Dc[k], u[k], acc);
        if (z != nullptr) y *= silu(zz[k]);
        out[(bb[k] * L + t) * dim + cc[k]] = from_f32<T>(y);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < R; ++k)
    if (live[k] && p.state_out != nullptr) storeS<S, VEC>(p.state_out + rr[k] * N, n0, N, h[k]);
  if constexpr (CONV) {   // the window after the last token (inputs, stored exactly as read)
    const int W = p.conv_width;
    T* cs = static_cast<T*>(p.conv_out);
#pragma unroll
    for (int k = 0; k < R; ++k)
      if (live[k] && n0 == 0 && cs != nullptr)
        for (int m = 1; m <= W - 1; ++m) cs[(bb[k] * (W - 1) + (W - 1 - m)) * dim + cc[k]] = from_f32<T>(win[k][3 - m]);
  }
}

// multi-head form: row = (b, h, p), state [batch, H, P, N]
template <typename T, bool VEC, int S, bool TRAP, bool ROT>
__global__ __launch_bounds__(kThreads) void ssd_update_kernel(UpdParams p) {
  static_assert(!ROT || (TRAP && S % 2 == 0), "the complex state comes with the trapezoidal rule, whole pairs");
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t row0 = gid / p.lpr;
  const int64_t rstride = static_cast<int64_t>(gridDim.x) * kThreads / p.lpr;
  const int n0 = S * static_cast<int>(gid % p.lpr);
  const int64_t P = p.P, H = p.H, G = p.G, L = p.L;
  const int N = static_cast<int>(p.N);
  const T* x = static_cast<const T*>(p.x);
  const T* delta = static_cast<const T*>(p.delta);
  const T* Bm = static_cast<const T*>(p.B);
  const T* Cm = static_cast<const T*>(p.C);
  const T* z = static_cast<const T*>(p.z);
  T* out = static_cast<T*>(p.out);

  bool live[R];
  int64_t rr[R], pp[R], hd[R], bb[R], gg[R];
  float h[R][S], a2[R], Dh[R];
  float up[R], bp[R][S];   // TRAP: the previous token's x (this row) and B (this lane's states)
  float om[R][S / 2];      // ROT: rotation rates of this lane's state pairs
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t row = row0 + k * rstride;
    live[k] = row < p.rows;
    rr[k] = live[k] ? row : 0;
    pp[k] = rr[k] % P;
    const int64_t bh = rr[k] / P;
    hd[k] = bh % H;
    bb[k] = bh / H;
    gg[k] = hd[k] / (H / G);
    if (p.state_in != nullptr) {
      loadS<S, VEC>(p.state_in + rr[k] * N, n0, N, h[k]);
    } else {
#pragma unroll
      for (int q = 0; q < S; ++q) h[k][q] = 0.f;
    }
    a2[k] = p.A[hd[k]] * kLog2e;
    Dh[k] = p.D != nullptr ? p.D[hd[k]] : 0.f;
    if constexpr (ROT) {
#pragma unroll
      for (int j = 0; j < S / 2; ++j) om[k][j] = n0 + 2 * j < N ? p.omega[hd[k] * (N / 2) + n0 / 2 + j] : 0.f;
    }
    if constexpr (TRAP) {
      up[k] = p.x_prev != nullptr ? to_f32(static_cast<const T*>(p.x_prev)[rr[k]]) : 0.f;   // rows are (b, h, p)
      if (p.B_prev != nullptr) {
        loadSio<T, S, VEC>(static_cast<const T*>(p.B_prev) + (bb[k] * G + gg[k]) * N, n0, N, bp[k]);
      } else {
#pragma unroll
        for (int q = 0; q < S; ++q) bp[k][q] = 0.f;
      }
    }
  }
  const T* lam = static_cast<const T*>(p.lam);
  for (int64_t t = 0; t < L; ++t) {
    float d[R], u[R], zz[R], lm[R], bv[R][S], cv[R][S];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int64_t obh = (bb[k] * L + t) * H + hd[k];
      d[k] = to_f32(delta[obh]);
      if constexpr (TRAP) lm[k] = to_f32(lam[obh]);
      u[k] = to_f32(x[obh * P + pp[k]]);
      zz[k] = z != nullptr ? to_f32(z[obh * P + pp[k]]) : 0.f;
      loadSio<T, S, VEC>(Bm + ((bb[k] * L + t) * G + gg[k]) * N, n0, N, bv[k]);
      loadSio<T, S, VEC>(Cm + ((bb[k] * L + t) * G + gg[k]) * N, n0, N, cv[k]);
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float dA = exp2_hw(d[k] * a2[k]), du = d[k] * u[k];
      float acc = 0.f;
      if constexpr (ROT) {
        // a R(d omega) (S + (1 - lam) d x_prev B_prev) + lam d x B, pair by pair
        const float wl = (1.f - lm[k]) * d[k] * up[k], wr = lm[k] * du;
#pragma unroll
        for (int j = 0; j < S / 2; ++j) {
          float sn, cs;
          sincos_rev(d[k] * om[k][j], sn, cs);
          const float tu = __builtin_fmaf(wl, bp[k][2 * j], h[k][2 * j]);
          const float tv = __builtin_fmaf(wl, bp[k][2 * j + 1], h[k][2 * j + 1]);
          const float ru = __builtin_fmaf(cs, tu, -(sn * tv)), rv = __builtin_fmaf(sn, tu, cs * tv);
          h[k][2 * j] = __builtin_fmaf(dA, ru, wr * bv[k][2 * j]);
          h[k][2 * j + 1] = __builtin_fmaf(dA, rv, wr * bv[k][2 * j + 1]);
        }
#pragma unroll
        for (int q = 0; q < S; ++q) {
          acc = __builtin_fmaf(cv[k][q], h[k][q], acc);
          bp[k][q] = bv[k][q];
        }
        up[k] = u[k];
      } else if constexpr (TRAP) {
        // a (S + (1 - lam) d x_prev B_prev) + lam d x B
        const float wl = (1.f - lm[k]) * d[k] * up[k], wr = lm[k] * du;
#pragma unroll
        for (int q = 0; q < S; ++q) {
          h[k][q] = __builtin_fmaf(dA, __builtin_fmaf(wl, bp[k][q], h[k][q]), wr * bv[k][q]);
          acc = __builtin_fmaf(cv[k][q], h[k][q], acc);
          bp[k][q] = bv[k][q];
        }
        up[k] = u[k];
      } else {
#pragma unroll
        for (int q = 0; q < S; ++q) {
          h[k][q] = __builtin_fmaf(dA, h[k][q], du * bv[k][q]);
          acc = __builtin_fmaf(cv[k][q], h[k][q], acc);
        }
      }
      acc = group_sum(acc, p.lpr);
      if (live[k] && n0 == 0) {
        float y = __builtin_fmaf(Dh[k], u[k], acc);
        if (z != nullptr) y *= silu(zz[k]);
        out[((bb[k] * L + t) * H + hd[k]) * P + pp[k]] = from_f32<T>(y);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < R; ++k)
    if (live[k] && p.state_out != nullptr) storeS<S, VEC>(p.state_out + rr[k] * N, n0, N, h[k]);
}

// Mamba-3 MIMO ("Mamba-3" blog, "El modelo Mamba-3" item 3), row = (b, h, p): the rank inputs of the
// row's channel drive its states through one transition, U = sum_r x_r B_r, and each rank reads them out
// through its own C_r.  Mamba-2 rule, or with TRAP the exponential-trapezoidal rule, whose left-end term
// uses the previous token's U.  The ranks are walked one at a time (S registers of B or C each).
template <typename T, bool VEC, int S, bool TRAP>
__global__ __launch_bounds__(kThreads) void ssdm_update_kernel(UpdParams p) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t row = gid / p.lpr;
  const int n0 = S * static_cast<int>(gid % p.lpr);
  const int64_t P = p.P, H = p.H, G = p.G, L = p.L, NR = p.rank;
  const int N = static_cast<int>(p.N);
  const T* x = static_cast<const T*>(p.x);
  const T* delta = static_cast<const T*>(p.delta);
  const T* Bm = static_cast<const T*>(p.B);
  const T* Cm = static_cast<const T*>(p.C);
  const T* z = static_cast<const T*>(p.z);
  T* out = static_cast<T*>(p.out);
  const bool live = row < p.rows;
  const int64_t rr = live ? row : 0;
  const int64_t pp = rr % P, bh = rr / P, hd = bh % H, bb = bh / H, gg = hd / (H / G);
  float h[S], up[S];
  if (p.state_in != nullptr) {
    loadS<S, VEC>(p.state_in + rr * N, n0, N, h);
  } else {
#pragma unroll
    for (int q = 0; q < S; ++q) h[q] = 0.f;
  }
  const float a2 = p.A[hd] * kLog2e;
  const float Dh = p.D != nullptr ? p.D[hd] : 0.f;
#pragma unroll
  for (int q = 0; q < S; ++q) up[q] = 0.f;   // TRAP: the previous token's sum_r x_r B_r
  if constexpr (TRAP) {
    if (p.x_prev != nullptr && p.B_prev != nullptr) {
      for (int64_t r = 0; r < NR; ++r) {
        float bv[S];
        const float u = to_f32(static_cast<const T*>(p.x_prev)[(bh * NR + r) * P + pp]);
        loadSio<T, S, VEC>(static_cast<const T*>(p.B_prev) + ((bb * G + gg) * NR + r) * N, n0, N, bv);
#pragma unroll
        for (int q = 0; q < S; ++q) up[q] = __builtin_fmaf(u, bv[q], up[q]);
      }
    }
  }
  const T* lam = static_cast<const T*>(p.lam);
  for (int64_t t = 0; t < L; ++t) {
    const int64_t obh = (bb * L + t) * H + hd;
    const int64_t bcr = ((bb * L + t) * G + gg) * NR;   // B, C row of rank 0
    const float d = to_f32(delta[obh]);
    const float dA = exp2_hw(d * a2);
    float U[S];
#pragma unroll
    for (int q = 0; q < S; ++q) U[q] = 0.f;
    for (int64_t r = 0; r < NR; ++r) {
      float bv[S];
      const float u = to_f32(x[(obh * NR + r) * P + pp]);
      loadSio<T, S, VEC>(Bm + (bcr + r) * N, n0, N, bv);
#pragma unroll
      for (int q = 0; q < S; ++q) U[q] = __builtin_fmaf(u, bv[q], U[q]);
    }
    if constexpr (TRAP) {
      const float lm = to_f32(lam[obh]);
      const float wl = (1.f - lm) * d, wr = lm * d;
#pragma unroll
      for (int q = 0; q < S; ++q) {
        h[q] = __builtin_fmaf(dA, __builtin_fmaf(wl, up[q], h[q]), wr * U[q]);
        up[q] = U[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < S; ++q) h[q] = __builtin_fmaf(dA, h[q], d * U[q]);
    }
    for (int64_t r = 0; r < NR; ++r) {
      float cv[S];
      loadSio<T, S, VEC>(Cm + (bcr + r) * N, n0, N, cv);
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < S; ++q) acc = __builtin_fmaf(cv[q], h[q], acc);
      acc = group_sum(acc, p.lpr);
      if (live && n0 == 0) {
        const int64_t o = (obh * NR + r) * P + pp;
        float y = __builtin_fmaf(Dh, to_f32(x[o]), acc);
        if (z != nullptr) y *= silu(to_f32(z[o]));
        out[o] = from_f32<T>(y);
      }
    }
  }
  if (live && p.state_out != nullptr) storeS<S, VEC>(p.state_out + rr * N, n0, N, h);
}

int lanes_per_row(int64_t N, int S) {
  int l = 1;
  while (static_cast<int64_t>(S) * l < N) l *= 2;
  return l;
}

UpdParams common(const UpdateArgs& a) {
  UpdParams p{};
  p.state = a.state; p.state_in = a.state != nullptr ? a.state : a.state_in;
  p.state_out = a.state != nullptr ? a.state : a.state_out;
  p.x = a.x; p.delta = a.delta; p.A = a.A; p.B = a.B; p.C = a.C; p.D = a.D; p.z = a.z;
  p.out = a.out;
  p.batch = a.batch; p.L = a.L; p.N = a.N;
  return p;
}

// vector accesses: whole groups of S states, 16-byte aligned state/A, B/C aligned to 4 elements
bool vec_ok(const UpdateArgs& a, bool mamba1, int S) {
  auto al = [](const void* q, uintptr_t m) { return (reinterpret_cast<uintptr_t>(q) & (m - 1)) == 0; };
  const uintptr_t bc = a.io == 1 ? 8 : 16;
  return a.N % S == 0 && al(a.state, 16) && al(a.state_in, 16) && al(a.state_out, 16) &&
         (!mamba1 || al(a.A, 16)) && al(a.B, bc) && al(a.C, bc) && (a.B_prev == nullptr || al(a.B_prev, bc));
}

int64_t grid_blocks(int64_t rows, int64_t N, int S) {
  // R rows per thread: the grid spans ceil(rows / R) rows of lanes
  return ((rows + R - 1) / R * lanes_per_row(N, S) + kThreads - 1) / kThreads;
}

// 8 states per lane when whole 8-groups fit (16 measured slower: fewer waves), else 4; the scalar
// path for other layouts
template <template <typename, bool, int> class K, typename T>
hipError_t launch_update(UpdParams p, const UpdateArgs& a, bool mamba1, hipStream_t stream) {
  if (vec_ok(a, mamba1, 8)) {
    p.lpr = lanes_per_row(a.N, 8);
    hipLaunchKernelGGL((K<T, true, 8>::fn), dim3(static_cast<unsigned>(grid_blocks(p.rows, a.N, 8))),
                       dim3(kThreads), 0, stream, p);
  } else {
    const bool vec = vec_ok(a, mamba1, 4);
    p.lpr = lanes_per_row(a.N, 4);
    const dim3 grid(static_cast<unsigned>(grid_blocks(p.rows, a.N, 4)));
    if (vec) hipLaunchKernelGGL((K<T, true, 4>::fn), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((K<T, false, 4>::fn), grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}
template <typename T, bool VEC, int S> struct ScanUpd { static constexpr auto fn = scan_update_kernel<T, VEC, S, false>; };
template <typename T, bool VEC, int S> struct ScanUpdConv { static constexpr auto fn = scan_update_kernel<T, VEC, S, true>; };
template <typename T, bool VEC, int S> struct SsdUpd { static constexpr auto fn = ssd_update_kernel<T, VEC, S, false, false>; };
template <typename T, bool VEC, int S> struct SsdUpdTrap { static constexpr auto fn = ssd_update_kernel<T, VEC, S, true, false>; };
template <typename T, bool VEC, int S> struct SsdUpdRot { static constexpr auto fn = ssd_update_kernel<T, VEC, S, true, true>; };
template <typename T, bool VEC, int S> struct SsdmUpd { static constexpr auto fn = ssdm_update_kernel<T, VEC, S, false>; };
template <typename T, bool VEC, int S> struct SsdmUpdTrap { static constexpr auto fn = ssdm_update_kernel<T, VEC, S, true>; };

}  // namespace

hipError_t scan_update_launch(const UpdateArgs& a, hipStream_t stream) {
  UpdParams p = common(a);
  p.dim = a.dim;
  p.rows = a.batch * a.dim;
  if (a.conv_w != nullptr) {
    p.conv_w = a.conv_w; p.conv_b = a.conv_b; p.conv_width = a.conv_width;
    p.conv_in = a.conv_state != nullptr ? a.conv_state : a.conv_in;
    p.conv_out = a.conv_state != nullptr ? a.conv_state : a.conv_out;
    return a.io == 1 ? launch_update<ScanUpdConv, uint16_t>(p, a, true, stream)
                     : launch_update<ScanUpdConv, float>(p, a, true, stream);
  }
  return a.io == 1 ? launch_update<ScanUpd, uint16_t>(p, a, true, stream)
                   : launch_update<ScanUpd, float>(p, a, true, stream);
}

hipError_t ssd_update_launch(const UpdateArgs& a, hipStream_t stream) {
  UpdParams p = common(a);
  p.H = a.H; p.P = a.P; p.G = a.G;
  p.rows = a.batch * a.H * a.P;
  p.rank = a.rank;
  if (a.rank > 1) {   // MIMO (no complex state)
    if (a.omega != nullptr) return hipErrorInvalidValue;
    if (a.lam != nullptr) {
      p.lam = a.lam; p.x_prev = a.x_prev; p.B_prev = a.B_prev;
      return a.io == 1 ? launch_update<SsdmUpdTrap, uint16_t>(p, a, false, stream)
                       : launch_update<SsdmUpdTrap, float>(p, a, false, stream);
    }
    return a.io == 1 ? launch_update<SsdmUpd, uint16_t>(p, a, false, stream)
                     : launch_update<SsdmUpd, float>(p, a, false, stream);
  }
  if (a.lam != nullptr) {
    p.lam = a.lam; p.x_prev = a.x_prev; p.B_prev = a.B_prev;
    if (a.omega != nullptr) {   // dstate is even: lanes own whole pairs (groups of 4 or 8 from a multiple of 4)
      p.omega = a.omega;
      return a.io == 1 ? launch_update<SsdUpdRot, uint16_t>(p, a, false, stream)
                       : launch_update<SsdUpdRot, float>(p, a, false, stream);
    }
    return a.io == 1 ? launch_update<SsdUpdTrap, uint16_t>(p, a, false, stream)
                     : launch_update<SsdUpdTrap, float>(p, a, false, stream);
  }
  return a.io == 1 ? launch_update<SsdUpd, uint16_t>(p, a, false, stream)
                   : launch_update<SsdUpd, float>(p, a, false, stream);
}

int64_t update_grid_blocks(int64_t rows, int64_t N) { return grid_blocks(rows, N, 4); }   // the largest grid

}  // namespace mssm
